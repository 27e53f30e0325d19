// gfx950 kernels for absorbed-MLA split-KV decode.
//
// Decode kernel.  One workgroup = 4 wavefronts = up to 128 query rows (query x head)
// of one request and one token range.  The workgroup streams the range's KV tiles
// (32 tokens x 576 values) from HBM straight into LDS with global->LDS loads (no
// register staging), dequantises FP8 / NVFP4 tiles in LDS to bf16, and each wavefront
// then runs, for its 32 rows:
//   S^T[32 tok x 32 rows] = KV_tile[32 x 576] . Q^T[576 x 32]       36 MFMA 32x32x16
//   masked online softmax over the tokens; a row lives in lanes l and l ^ 32
//   O^T[512 x 32] += V^T[512 x 32 tok] . P^T[32 tok x 32 rows]       32 MFMA 32x32x16
// Q^T stays in registers for the whole range and O^T accumulates in registers.  V^T
// operands come from the token-major tile through the LDS transpose read.  All heads
// of a request share one latent (absorbed MLA), so they all run against the same LDS
// tile (the TileGym page's kernel re-reads the tile once per group of 16 heads).
// Pipeline: raw tiles are loaded two tiles ahead of the MFMA work and dequantised one
// tile ahead, with one workgroup barrier per tile.
//
// Combine kernels.  One wavefront per output row merges the partials with the split-K
// log-sum-exp reduce (TileGym page, forward: splitk_reduce).

#include "mla_internal.h"

#include <math.h>

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int kKSteps = kRow / 16;                        // 36 K-steps of 16 for QK
constexpr int kRowChunks = kRow * 2 / 16;                 // 72 bf16 chunks of 16 B per token
constexpr int kTileRowBytes = kRowChunks * 16;            // 1152
constexpr int kTileBytes = kTileTokens * kTileRowBytes;   // 36864
constexpr int kDimBlocks = kLatent / 32;                  // 16 output blocks of 32 dims
constexpr int kFp8Chunks = kTileTokens * (kRow / 16);     // 1152 chunks of 16 codes
constexpr int kNvDataBytes = kRow / 2;                    // 288 packed E2M1 bytes per token
constexpr int kNvScaleBytes = kRow / 16;                  // 36 E4M3 scales per token
constexpr int kNvChunks = kTileTokens * kNvDataBytes / 16;        // 576
constexpr int kNvScaleWords = kTileTokens * kNvScaleBytes / 4;    // 288
constexpr int kNvStageData = kTileTokens * kNvDataBytes;          // 9216
constexpr float kTau = 8.0f;   // lazy rescale threshold (log2 units)
constexpr float kLn2 = 0.69314718055994531f;

template <int FMT>
struct StageBytes {
  static constexpr int value = FMT == kFmtFp8 ? kFp8Chunks * 16
                               : FMT == kFmtNvfp4 ? kNvStageData + kTileTokens * kNvScaleBytes
                                                  : 16;
};

// Byte offset of 16-byte chunk c (0..71) of token row r in a bf16 tile.  The chunk
// index is XOR-swizzled inside its aligned group of 8 (72 = 9 x 8) so that MFMA operand
// reads of consecutive token rows, 1152 B apart, spread over the LDS banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int tile_off(int r, int c) { return r * kTileRowBytes + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ unsigned pack_hi16(float lo, float hi) {
  // bf16 pair from two floats whose low 16 bits are zero (exact conversion)
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

// Four E4M3 codes (one dword) -> four bf16 (two dwords), exactly.
__device__ __forceinline__ void fp8x4_to_bf16(unsigned w, unsigned& o0, unsigned& o1) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o0 = pack_hi16(a[0], a[1]);
  o1 = pack_hi16(b[0], b[1]);
}

// E2M1 code (low 4 bits) -> float: 0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign.
__device__ __forceinline__ float e2m1_to_f32(unsigned c) {
  unsigned m = c & 7u;
  float mag = (m >= 2u) ? __uint_as_float((m << 22) + 0x3F000000u) : (m ? 0.5f : 0.0f);
  return (c & 8u) ? -mag : mag;
}

// Eight E2M1 codes (one dword, even value in the low nibble) times one scale -> eight
// bf16 (four dwords).  The products have at most 6 significant bits: exact in bf16.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(unsigned w, float s) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = e2m1_to_f32(w >> (8 * i)) * s;
    float hi = e2m1_to_f32(w >> (8 * i + 4)) * s;
    out[i] = pack_hi16(lo, hi);
  }
  return out;
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Combine the values of lanes l and l ^ 32 with one cross-half lane swap: r[0] holds the
// low half's value in both halves, r[1] the high half's.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// 16 bytes (or 4) per lane from global memory into LDS at lds_base + lane * size; the
// LDS base is the same for the whole wavefront.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const GLB_AS void*)g, (LDS_AS void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const GLB_AS void*)g, (LDS_AS void*)lds_base, 4, 0, 0);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------------------------
// Tile sources.  Tokens past the end of the request are clamped to its last token
// (their scores are masked, and a real row keeps every value finite); a 32-token tile
// never crosses a page (page sizes 32 and 64), so one block-table entry serves a tile.
// ------------------------------------------------------------------------------------

struct Range {
  const DecodeParams* p;
  int b;   // request
  int n;   // its tokens
};

__device__ __forceinline__ const uint8_t* tile_page(const Range& R, int tbase) {
  const DecodeParams& p = *R.p;
  int page = p.block_tables[(int64_t)R.b * p.max_blocks + tbase / p.page_size];
  page = min(max(page, 0), p.num_pages - 1);
  return p.cache + (int64_t)page * p.page_stride;
}

// bf16 rows straight into the swizzled tile: LDS chunk position q of row r holds
// logical chunk q ^ swz(r).  2304 chunks = 36 wave loads, 9 per wavefront.
template <bool PAGED>
__device__ __forceinline__ void load_bf16_tile(const Range& R, int tbase, uint8_t* tile, int wave, int lane) {
  const DecodeParams& p = *R.p;
  const uint8_t* pg = PAGED ? tile_page(R, tbase) : nullptr;
#pragma unroll
  for (int jj = 0; jj < kTileTokens * kRowChunks / 64 / kWaves; ++jj) {
    const int j = wave + kWaves * jj;
    const int k = 64 * j + lane;
    const int r = k / kRowChunks, pos = k % kRowChunks;
    const int c = pos ^ swz(r);
    const int tok = min(tbase + r, R.n - 1);
    const void* src;
    if (PAGED) {
      src = pg + (int64_t)(tok % p.page_size) * (2 * kRow) + 16 * c;
    } else {
      const int64_t t = (int64_t)R.b * p.S + tok;
      src = (c < kLatent / 8) ? (const void*)(p.kv + t * kLatent + 8 * c)
                              : (const void*)(p.kpe + t * kRope + 8 * (c - kLatent / 8));
    }
    dma16(src, tile + 1024 * j);
  }
}

// FP8 rows, raw, into staging [32][576]: 18 wave loads.
__device__ __forceinline__ void load_fp8_raw(const Range& R, int tbase, uint8_t* st, int wave, int lane) {
  const DecodeParams& p = *R.p;
  const uint8_t* pg = tile_page(R, tbase);
  for (int j = wave; j < kFp8Chunks / 64; j += kWaves) {
    const int k = 64 * j + lane;
    const int r = k / (kRow / 16), c = k % (kRow / 16);
    const int tok = min(tbase + r, R.n - 1);
    dma16(pg + (int64_t)(tok % p.page_size) * kRow + 16 * c, st + 1024 * j);
  }
}

// NVFP4 rows, raw: data [32][288] (9 wave loads of 16 B), then scales [32][36]
// (5 wave loads of 4 B, the last one half masked).
__device__ __forceinline__ void load_nvfp4_raw(const Range& R, int tbase, uint8_t* st, int wave, int lane) {
  const DecodeParams& p = *R.p;
  const uint8_t* pg = tile_page(R, tbase);
  for (int j = wave; j < kNvChunks / 64; j += kWaves) {
    const int k = 64 * j + lane;
    const int r = k / (kNvDataBytes / 16), c = k % (kNvDataBytes / 16);
    const int tok = min(tbase + r, R.n - 1);
    dma16(pg + (int64_t)(tok % p.page_size) * kNvDataBytes + 16 * c, st + 1024 * j);
  }
  const uint8_t* sc = pg + (int64_t)p.page_size * kNvDataBytes;
  for (int j = wave; j < (kNvScaleWords + 63) / 64; j += kWaves) {
    const int d = 64 * j + lane;
    if (d < kNvScaleWords) {
      const int r = d / (kNvScaleBytes / 4), c = d % (kNvScaleBytes / 4);
      const int tok = min(tbase + r, R.n - 1);
      dma4(sc + (int64_t)(tok % p.page_size) * kNvScaleBytes + 4 * c, st + kNvStageData + 256 * j);
    }
  }
}

// Raw staging -> bf16 tile.
__device__ __forceinline__ void dequant_fp8(const uint8_t* st, uint8_t* tile, int tid) {
#pragma unroll
  for (int j = 0; j < (kFp8Chunks + kThreads - 1) / kThreads; ++j) {
    const int k = tid + kThreads * j;
    if (k < kFp8Chunks) {
      const int r = k / (kRow / 16), c = k % (kRow / 16);
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + 16 * k);
      unsigned t[8];
      fp8x4_to_bf16(v[0], t[0], t[1]);
      fp8x4_to_bf16(v[1], t[2], t[3]);
      fp8x4_to_bf16(v[2], t[4], t[5]);
      fp8x4_to_bf16(v[3], t[6], t[7]);
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 2 * c)) = u32x4{t[0], t[1], t[2], t[3]};
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 2 * c + 1)) = u32x4{t[4], t[5], t[6], t[7]};
    }
  }
}

__device__ __forceinline__ void dequant_nvfp4(const uint8_t* st, uint8_t* tile, int tid) {
#pragma unroll
  for (int j = 0; j < (kNvChunks + kThreads - 1) / kThreads; ++j) {
    const int k = tid + kThreads * j;
    if (k < kNvChunks) {
      const int r = k / (kNvDataBytes / 16), c = k % (kNvDataBytes / 16);
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + 16 * k);
      const unsigned short sc =
          *reinterpret_cast<const unsigned short*>(st + kNvStageData + r * kNvScaleBytes + 2 * c);
      const f32x2 s = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc, false);
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 4 * c + 0)) = fp4x8_to_bf16(v[0], s[0]);
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 4 * c + 1)) = fp4x8_to_bf16(v[1], s[0]);
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 4 * c + 2)) = fp4x8_to_bf16(v[2], s[1]);
      *reinterpret_cast<u32x4*>(tile + tile_off(r, 4 * c + 3)) = fp4x8_to_bf16(v[3], s[1]);
    }
  }
}

// ------------------------------------------------------------------------------------
// Per-wavefront attention state and the work on one tile
// ------------------------------------------------------------------------------------

struct WaveState {
  bf16x8 q[kKSteps];        // Q^T operand: row lr, dims 16k + 8lh .. +8
  f32x16 o[kDimBlocks];     // O^T accumulators: row lr, dims 32d + 8(v/4) + 4lh + v%4
  float m_used;             // reference max (log2 domain), equal in lanes l and l^32
  float l_sum;              // this lane's share of sum p (unrounded): for the LSE
  float l_rnd;              // this lane's share of sum bf16(p): normalises O
  int qk_off[4];            // LDS byte offsets of the QK operand, K-step k -> [k & 3] + 128 (k >> 2)
  int pv_off[8];            // LDS byte offsets of the V^T transpose reads
  int vis;                  // tokens this lane's row may see
};

__device__ __forceinline__ void mm_tile(WaveState& W, const uint8_t* tile, int tbase, float score_scale, int lh) {
  // ---- S^T = KV . Q^T: lane holds row lr, tokens 8(v/4) + 4lh + v%4 ----
  f32x16 s = f32x16{};
#pragma unroll
  for (int k = 0; k < kKSteps; ++k) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(tile + W.qk_off[k & 3] + 128 * (k >> 2));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, W.q[k], s, 0, 0, 0);
  }

  // ---- mask + online softmax (base 2) ----
  float mt = -INFINITY;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int tok = tbase + 8 * (v >> 2) + 4 * lh + (v & 3);
    const float x = (tok < W.vis) ? s[v] * score_scale : -INFINITY;
    s[v] = x;
    mt = fmaxf(mt, x);
  }
  mt = pair_max(mt);
  const bool need = mt > W.m_used + kTau;
  if (__any(need)) {
    const float m_new = need ? mt : W.m_used;
    const float alpha = need ? __builtin_amdgcn_exp2f(W.m_used - m_new) : 1.0f;
    W.l_sum *= alpha;
    W.l_rnd *= alpha;
#pragma unroll
    for (int d = 0; d < kDimBlocks; ++d) W.o[d] *= alpha;
    W.m_used = m_new;
  }
  const float msafe = (W.m_used == -INFINITY) ? 0.f : W.m_used;
  bf16x8 pb[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float e = __builtin_amdgcn_exp2f(s[v] - msafe);
    W.l_sum += e;
    const __bf16 eb = (__bf16)e;
    W.l_rnd += (float)eb;
    pb[v >> 3][v & 7] = eb;
  }

  // ---- O^T += V^T . P^T; K index e of K-step ks <-> token 16ks + 8(e/4) + 4lh + e%4 ----
#pragma unroll
  for (int d = 0; d < kDimBlocks; ++d) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o0 = W.pv_off[4 * (d & 1) + 2 * ks + 0] + 128 * (d >> 1);
      const int o1 = W.pv_off[4 * (d & 1) + 2 * ks + 1] + 128 * (d >> 1);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o1));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      W.o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], W.o[d], 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------------------------------
// One token range of one request: Q load, pipelined tile loop, partial epilogue
// ------------------------------------------------------------------------------------

template <int FMT, bool PAGED>
__device__ __forceinline__ void run_range(const DecodeParams& p, uint8_t* bf0, uint8_t* bf1, uint8_t* st0,
                                          uint8_t* st1, int b, int n, int rg, int lt0, int lt1, int64_t slot) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int row_w0 = rg * kRowsPerGroup + wave * kRowsPerWave;  // first row of this wave
  const bool active = row_w0 < p.rows;
  const int row = row_w0 + lr;
  const int rc = min(row, p.rows - 1);

  WaveState W;
  W.vis = max(n - p.q_len + rc / p.H + 1, 0);
  W.m_used = -INFINITY;
  W.l_sum = 0.f;
  W.l_rnd = 0.f;
  {
    const uint16_t* qrow = p.q + ((int64_t)b * p.rows + rc) * kLatent;
    const uint16_t* prow = p.qpe + ((int64_t)b * p.rows + rc) * kRope;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const uint16_t* src = (k < kLatent / 16) ? qrow + 16 * k + 8 * lh : prow + 16 * (k - kLatent / 16) + 8 * lh;
      W.q[k] = *reinterpret_cast<const bf16x8*>(src);
    }
  }
#pragma unroll
  for (int d = 0; d < kDimBlocks; ++d) W.o[d] = f32x16{};
  // QK operand: token lr, logical chunk 2k + lh.  (2k + lh) ^ s = 8(k >> 2) + ((2(k & 3) + lh) ^ s).
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) W.qk_off[kk] = lr * kTileRowBytes + (((2 * kk + lh) ^ swz(lr)) << 4);
  // V^T transpose reads: in a group of 16 lanes (g = lane / 16, j = lane % 16), lane j
  // addresses token 16ks + 8e + 4(g >> 1) + j / 4 and dims 32d + 16(g & 1) + 4(j % 4)..+4;
  // lane i of the group then receives dim 32d + 16(g & 1) + i of those four tokens.
  {
    const int g = lane >> 4, j = lane & 15;
    const int dlo = 16 * (g & 1) + 4 * (j & 3);  // dim inside the 32-dim block
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tok = 16 * ks + 8 * e + 4 * (g >> 1) + (j >> 2);
          const int dim = 32 * dp + dlo;
          W.pv_off[4 * dp + 2 * ks + e] = tile_off(tok, dim >> 3) + 2 * (dim & 7);
        }
  }
  const float score_scale = p.score_scale;
  const int nt = lt1 - lt0;
  Range R{&p, b, n};

  if (nt > 0) {
    if (FMT == kFmtBf16) {
      // raw bf16 rows go straight into the two tiles; loads run one tile ahead
      load_bf16_tile<PAGED>(R, lt0 * kTileTokens, bf0, wave, lane);
      for (int i = 0;;) {
        wait_dma();
        __syncthreads();
        if (i + 1 < nt) load_bf16_tile<PAGED>(R, (lt0 + i + 1) * kTileTokens, bf1, wave, lane);
        if (active) mm_tile(W, bf0, (lt0 + i) * kTileTokens, score_scale, lh);
        if (++i >= nt) break;
        wait_dma();
        __syncthreads();
        if (i + 1 < nt) load_bf16_tile<PAGED>(R, (lt0 + i + 1) * kTileTokens, bf0, wave, lane);
        if (active) mm_tile(W, bf1, (lt0 + i) * kTileTokens, score_scale, lh);
        if (++i >= nt) break;
      }
    } else {
      // raw tiles two ahead of the MFMA work, dequantised one ahead
      auto load_raw = [&](int i, uint8_t* st) {
        if (FMT == kFmtFp8) load_fp8_raw(R, (lt0 + i) * kTileTokens, st, wave, lane);
        else load_nvfp4_raw(R, (lt0 + i) * kTileTokens, st, wave, lane);
      };
      auto dequant = [&](const uint8_t* st, uint8_t* tile) {
        if (FMT == kFmtFp8) dequant_fp8(st, tile, tid);
        else dequant_nvfp4(st, tile, tid);
      };
      load_raw(0, st0);
      if (nt > 1) load_raw(1, st1);
      wait_dma();
      __syncthreads();
      dequant(st0, bf0);
      for (int i = 0;;) {
        wait_dma();
        __syncthreads();
        if (i + 2 < nt) load_raw(i + 2, st0);
        if (i + 1 < nt) dequant(st1, bf1);
        if (active) mm_tile(W, bf0, (lt0 + i) * kTileTokens, score_scale, lh);
        if (++i >= nt) break;
        wait_dma();
        __syncthreads();
        if (i + 2 < nt) load_raw(i + 2, st1);
        if (i + 1 < nt) dequant(st0, bf0);
        if (active) mm_tile(W, bf1, (lt0 + i) * kTileTokens, score_scale, lh);
        if (++i >= nt) break;
      }
    }
  }
  __syncthreads();  // the next range reuses the buffers

  // ---- epilogue: normalised partial and its log-sum-exp ----
  if (active) {
    const float l_tot = pair_sum(W.l_sum);
    const float l_rnd = pair_sum(W.l_rnd);
    const bool ok = l_tot > 0.f;
    const float inv = ok ? p.v_scale / l_rnd : 0.f;
    const float lse = ok ? (W.m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (row < p.rows) {
      float* orow = p.o_part + slot * p.o_slot + (int64_t)row * p.o_row;
#pragma unroll
      for (int d = 0; d < kDimBlocks; ++d) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 val = {W.o[d][4 * g] * inv, W.o[d][4 * g + 1] * inv, W.o[d][4 * g + 2] * inv,
                             W.o[d][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * d + 8 * g + 4 * lh) = val;
        }
      }
      if (lh == 0) p.lse_part[slot * p.l_slot + (int64_t)row * p.l_row] = lse;
    }
  }
}

// ------------------------------------------------------------------------------------
// decode kernels
// ------------------------------------------------------------------------------------

// Contiguous: grid (row_groups, num_splits, B); split j covers [j*L, min((j+1)*L, S)).
__global__ __launch_bounds__(kThreads) void decode_contig_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t bf0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bf1[kTileBytes];
  const int rg = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t0 = j * p.kv_len_per_split;
  const int t1 = min(t0 + p.kv_len_per_split, p.S);
  const int lt0 = t0 / kTileTokens;
  const int lt1 = (t1 + kTileTokens - 1) / kTileTokens;
  // slot b*H*NS + j with row = head addresses o_part [B, H, NS, 512]
  run_range<kFmtBf16, false>(p, bf0, bf1, nullptr, nullptr, b, p.S, rg, lt0, lt1,
                             (int64_t)b * p.rows * p.num_splits + j);
}

// Paged: the batch's tiles (request b has ceil(n_b / 32)) are cut into num_splits equal
// ranges, range w -> workgroup w (x row_groups).  A range covering parts of several
// requests runs one segment per request; segment (w, b) writes partial slot w + b,
// unique because the ranges are ordered.  seg_first[b] / seg_last[b] record the first
// and last range touching request b; info[0] records the total tile count.
template <int FMT>
__global__ __launch_bounds__(kThreads) void decode_paged_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t bf0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bf1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st0[StageBytes<FMT>::value];
  __shared__ __attribute__((aligned(16))) uint8_t st1[StageBytes<FMT>::value];
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int max_len = p.max_blocks * p.page_size;

  // workgroup id -> (range w, row group rg); the row groups of one range sit 8 ids
  // apart so that they land on the same XCD (ids are dealt round-robin over 8 XCDs)
  const int id = blockIdx.x;
  const int per_blk = 8 * p.row_groups;
  const int rg = (id % per_blk) / 8;
  const int w = (id / per_blk) * 8 + (id % 8);
  if (w >= p.num_splits) return;

  // exclusive prefix of tile counts over requests -> pre[0..B]
  {
    const int per = (p.B + kThreads - 1) / kThreads;
    const int s0 = min(tid * per, p.B), s1 = min(s0 + per, p.B);
    int acc = 0;
    for (int b = s0; b < s1; ++b) {
      const int n = min(max(p.seq_lens[b], 0), max_len);
      acc += (n + kTileTokens - 1) / kTileTokens;
    }
    int x = acc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int run = x - acc;
    for (int i = 0; i < wave; ++i) run += wsum[i];
    if (tid == 0) pre[0] = 0;
    for (int b = s0; b < s1; ++b) {
      const int n = min(max(p.seq_lens[b], 0), max_len);
      run += (n + kTileTokens - 1) / kTileTokens;
      pre[b + 1] = run;
    }
    __syncthreads();
  }

  const int T = pre[p.B];
  if (w == 0 && rg == 0 && tid == 0) p.info[0] = T;
  const int t0 = (int)(((int64_t)w * T) / p.num_splits);
  const int t1 = (int)(((int64_t)(w + 1) * T) / p.num_splits);
  if (t0 >= t1) return;

  // request holding tile t0: the last b with pre[b] <= t0
  int lo = 0, hi = p.B;  // pre[lo] <= t0 < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= t0) lo = mid; else hi = mid;
  }
  int b = lo;
  int t = t0;
  while (t < t1) {
    while (pre[b + 1] <= t) ++b;  // skip empty requests
    const int seg_end = min(t1, pre[b + 1]);
    const int n = min(max(p.seq_lens[b], 0), max_len);
    run_range<FMT, true>(p, bf0, bf1, st0, st1, b, n, rg, t - pre[b], seg_end - pre[b], (int64_t)w + b);
    if (tid == 0 && rg == 0) {
      if (t == pre[b]) p.seg_first[b] = w;
      if (seg_end == pre[b + 1]) p.seg_last[b] = w;
    }
    t = seg_end;
    ++b;
  }
}

// ------------------------------------------------------------------------------------
// combine kernels (one wavefront per output row)
// ------------------------------------------------------------------------------------

struct PartRef {
  float lse;
  const float* o;
};

// Merge ns partials of one row; part(j) returns (lse_j, pointer to O_j).
template <class Part>
__device__ __forceinline__ void combine_row(int ns, Part part, uint16_t* orow, float* lse_out, int lane) {
  float M = -INFINITY;
  for (int j = lane; j < ns; j += 64) M = fmaxf(M, part(j).lse);
  M = wave_max(M);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float LSE = -INFINITY;
  if (M != -INFINITY) {
    float den = 0.f;
    for (int j = lane; j < ns; j += 64) den += expf(part(j).lse - M);
    den = wave_sum(den);
    LSE = M + logf(den);
    for (int j = 0; j < ns; ++j) {
      const PartRef pj = part(j);
      if (pj.lse == -INFINITY) continue;
      const float wgt = expf(pj.lse - LSE);
      const f32x4* src = reinterpret_cast<const f32x4*>(pj.o + 8 * lane);
      const f32x4 a = src[0], c = src[1];
      acc[0] += wgt * a[0]; acc[1] += wgt * a[1]; acc[2] += wgt * a[2]; acc[3] += wgt * a[3];
      acc[4] += wgt * c[0]; acc[5] += wgt * c[1]; acc[6] += wgt * c[2]; acc[7] += wgt * c[3];
    }
  }
  u32x4 packed;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    packed[i] = (unsigned)f32_to_bf16_rne(acc[2 * i]) | ((unsigned)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(orow + 8 * lane) = packed;
  if (lse_out && lane == 0) *lse_out = LSE;
}

// generic: o_part [rows, ns, 512], lse_part [rows, ns]
__global__ __launch_bounds__(256) void combine_generic_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const float* lses = p.lse_part + row * p.num_splits;
  const float* base = p.o_part + row * p.num_splits * kLatent;
  auto part = [&](int j) { return PartRef{lses[j], base + (int64_t)j * kLatent}; };
  combine_row(p.num_splits, part, p.o + row * kLatent, p.lse ? p.lse + row : nullptr, lane);
}

// paged: row (b, r) merges slots w + b for the non-empty ranges w in
// [seg_first[b], seg_last[b]]; o_part [slots, rows, 512], lse_part [slots, rows]
__global__ __launch_bounds__(256) void combine_paged_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grow >= (int64_t)p.B * p.rows) return;
  const int b = (int)(grow / p.rows), r = (int)(grow % p.rows);
  const int n = min(max(p.seq_lens[b], 0), p.max_len);
  const int T = p.info[0];
  const int G = p.num_splits;
  int w0 = 0, w1 = -1;
  if (n > 0) {  // descriptors written by the decode launch; clamped so they never address outside
    w0 = min(max(p.seg_first[b], 0), G - 1);
    w1 = min(max(p.seg_last[b], w0), G - 1);
  }
  auto part = [&](int j) {
    const int wj = w0 + j;
    const bool live = ((int64_t)wj * T) / G < ((int64_t)(wj + 1) * T) / G;  // range wj holds tiles
    const int64_t slot = (int64_t)wj + b;
    return PartRef{live ? p.lse_part[slot * p.rows + r] : -INFINITY, p.o_part + (slot * p.rows + r) * kLatent};
  };
  combine_row(w1 - w0 + 1, part, p.o + grow * kLatent, p.lse ? p.lse + grow : nullptr, lane);
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------

hipError_t launch_decode_contig(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.row_groups, p.num_splits, p.B);
  hipLaunchKernelGGL(decode_contig_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_paged(int fmt, const DecodeParams& p, hipStream_t stream) {
  const int blocks = ((p.num_splits + 7) / 8) * 8 * p.row_groups;
  switch (fmt) {
    case kFmtBf16:
      hipLaunchKernelGGL(decode_paged_kernel<kFmtBf16>, dim3(blocks), dim3(kThreads), 0, stream, p);
      break;
    case kFmtFp8:
      hipLaunchKernelGGL(decode_paged_kernel<kFmtFp8>, dim3(blocks), dim3(kThreads), 0, stream, p);
      break;
    case kFmtNvfp4:
      hipLaunchKernelGGL(decode_paged_kernel<kFmtNvfp4>, dim3(blocks), dim3(kThreads), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine_generic(const CombineParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(combine_generic_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine_paged(const CombineParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.rows;
  hipLaunchKernelGGL(combine_paged_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
