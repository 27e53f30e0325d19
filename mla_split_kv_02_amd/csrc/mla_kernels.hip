// gfx950 kernels for absorbed-MLA split-KV decode.
//
// Decode kernel.  One workgroup = 8 wavefronts (two per SIMD) = up to 128 query rows
// (query x head) of one request and one token range.  The workgroup streams the
// range's KV tiles (32 tokens x 576 values) from HBM straight into LDS with global->LDS
// loads (no register staging) and dequantises FP8 / NVFP4 tiles in LDS to bf16.  Each
// tile then takes two phases separated by a workgroup barrier:
//   scores:  wavefront w computes S^T[32 tok x 16 rows] for rows 16w..16w+15 with MFMA
//            16x16x32 (its Q^T rows stay in registers), applies the mask and the online
//            softmax, and publishes P (bf16) and the rows' rescale factors in LDS;
//   output:  wavefront w accumulates O^T[64 dims x 128 rows] for dims 64w..64w+63 with
//            MFMA 32x32x16, V^T read from the token-major tile with the LDS transpose
//            load and P^T from LDS.
// All heads of a request share one latent (absorbed MLA), so every row of the group
// runs against the same LDS tile (the TileGym page's kernel instead re-reads the tile
// once per group of 16 heads).
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
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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
// Tile sources.  Every global->LDS load instruction runs on all 64 lanes and moves 64
// consecutive 16-byte chunks of the tile.  Tokens past the end of the request are clamped
// to its last token (their scores are masked, and a real row keeps every value finite);
// a 32-token tile never crosses a page (page sizes 32 and 64), so one block-table entry
// serves a tile.
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
  for (int j = wave; j < kTileTokens * kRowChunks / 64; j += kWaves) {
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

// Four E4M3 codes (one dword) -> four bf16 (two dwords), exactly (hardware convert with
// unit scale).
__device__ __forceinline__ void fp8x4_to_bf16(unsigned w, unsigned& o0, unsigned& o1) {
  o0 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
  o1 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
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
// Work split inside a workgroup (8 wavefronts, 128 query rows).
//   Score phase: wavefront w owns rows 16w .. 16w+15.  S^T[32 tok x 16 rows] from
//     18 K-steps x 2 token blocks of MFMA 16x16x32 (Q^T of its rows in registers), then
//     the masked online softmax; P (bf16) and each row's rescale factor go to LDS.
//   Output phase: wavefront w owns dims 64w .. 64w+63 of all 128 rows:
//     O^T[64 x 128] += V^T[64 x 32 tok] . P^T[32 tok x 128] with MFMA 32x32x16, V^T
//     through the LDS transpose read of the token-major tile, P^T from LDS.
// Two wavefronts share a SIMD, so one's MFMA work overlaps the other's softmax and
// loads, and every wavefront stays within 256 registers.
// ------------------------------------------------------------------------------------

constexpr int kQkSteps = kRow / 32;          // 18 K-steps of 32 dims (MFMA 16x16x32)
constexpr int kPRowPitch = 80;               // bytes per row of the P buffer (64 + 16 pad)
constexpr int kPBufBytes = kRowsPerGroup * kPRowPitch;

struct Shared {  // LDS exchanged between the two phases of a tile
  uint8_t* pbuf;  // P as bf16 [128 rows][32 tokens], row pitch kPRowPitch
  float* alpha;   // [128] factor for each row's accumulators before this tile's product
  float* inv_l;   // [128] at the end of a range: v_scale / sum of bf16(p) (0 if no token)
};

struct ScoreState {
  bf16x8 q[kQkSteps];  // Q^T operand: row 16w + l%16, dims 32k + 8(l/16) .. +8
  float m_used;        // reference max (log2 domain), equal in the 4 lanes of a row
  float l_sum;         // this lane's share of sum p (unrounded): for the LSE
  float l_rnd;         // this lane's share of sum bf16(p): normalises O
  int vis;             // tokens the row may see
  int a_off;           // KV operand offset of token l%16, chunk l/16 (K-step 0, token block 0);
                       // K-step k: ^ 64 (k & 1), + 128 (k >> 1); token block 1: + 16 rows
  int p_off;           // P write offset: row * pitch + 8 (l / 16), + 32 tb
};

struct OutState {
  f32x16 o[2][4];      // o[db][rb]: row 32rb + l%32, dims 64w + 32db + 8(v/4) + 4(l/32) + v%4
  int v_off[2];        // transpose-read offsets for e = 0, 1 (db = 0, ks = 0); db = 1: ^ 64,
                       // ks = 1: + 16 rows
  int p_off;           // P^T operand: row l%32, tokens 16ks + 8(l/32): + 32*pitch*rb + 32 ks
};

// Values of the four lanes l, l^16, l^32, l^48 (one row), combined with lane swaps.
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return pair_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return pair_sum(x);
}

// Score phase of one tile for this wavefront's 16 rows.  `full`: every token of the tile
// is visible to every row of this wavefront, so no mask is needed.  c = score scale
// (log2 units, >= 0).
__device__ __forceinline__ void score_tile(ScoreState& S, const uint8_t* tile, const Shared& X, int tbase, float c,
                                           int lane, bool active, bool full, int row_in_group) {
  const int g = lane >> 4;
  f32x4 s0 = f32x4{}, s1 = f32x4{};
  if (active) {
#pragma unroll
    for (int k = 0; k < kQkSteps; ++k) {
      const int off = (S.a_off ^ (64 * (k & 1))) + 128 * (k >> 1);
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(tile + off);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(tile + off + 16 * kTileRowBytes);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, S.q[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, S.q[k], s1, 0, 0, 0);
    }
  }
  // lane holds row l%16, raw scores of tokens tbase + 16 tb + 4(l/16) + v
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  const int lim = S.vis - tbase - 4 * g;  // token j of this lane (16 tb + v) is visible iff j < lim
  if (!full) {
#pragma unroll
    for (int v = 0; v < 8; ++v) x[v] = (16 * (v >> 2) + (v & 3) < lim) ? x[v] : -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mt = quad_max(mt);
  mt = (mt == -INFINITY) ? -INFINITY : mt * c;
  const bool need = mt > S.m_used + kTau;
  float alpha = 1.0f;
  if (__any(need)) {
    const float m_new = need ? mt : S.m_used;
    alpha = need ? __builtin_amdgcn_exp2f(S.m_used - m_new) : 1.0f;
    S.l_sum *= alpha;
    S.l_rnd *= alpha;
    S.m_used = m_new;
  }
  const float nm = (S.m_used == -INFINITY) ? 0.f : -S.m_used;
  float e[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) e[v] = __builtin_amdgcn_exp2f(fmaf(x[v], c, nm));
  if (!full) {
#pragma unroll
    for (int v = 0; v < 8; ++v) e[v] = (16 * (v >> 2) + (v & 3) < lim) ? e[v] : 0.f;
  }
  S.l_sum += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  unsigned pk[4];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const bf16x2 pr = {(__bf16)e[2 * v], (__bf16)e[2 * v + 1]};
    S.l_rnd = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, S.l_rnd, false);
    pk[v] = __builtin_bit_cast(unsigned, pr);
  }
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  *reinterpret_cast<u32x2*>(X.pbuf + S.p_off) = u32x2{pk[0], pk[1]};
  *reinterpret_cast<u32x2*>(X.pbuf + S.p_off + 32) = u32x2{pk[2], pk[3]};
  if (g == 0) X.alpha[row_in_group] = alpha;
}

// Output phase of one tile for this wavefront's 64 dims of the first nrb row blocks;
// `side` is independent work (the next tile's dequantisation) issued between the MFMAs.
template <class Side>
__device__ __forceinline__ void out_tile(OutState& O, const uint8_t* tile, const Shared& X, int nrb, int lane,
                                         Side side) {
  const int lr = lane & 31;
  float al[4];
  bool resc = false;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    al[rb] = (rb < nrb) ? X.alpha[32 * rb + lr] : 1.0f;
    resc |= al[rb] != 1.0f;
  }
  if (__any(resc)) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      O.o[0][rb] *= al[rb];
      O.o[1][rb] *= al[rb];
    }
  }
  side();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 va[2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int o0 = (O.v_off[0] ^ (64 * db)) + 16 * kTileRowBytes * ks;
      const int o1 = (O.v_off[1] ^ (64 * db)) + 16 * kTileRowBytes * ks;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o1));
      va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb < nrb) {
        const bf16x8 pb = *reinterpret_cast<const bf16x8*>(X.pbuf + O.p_off + 32 * kPRowPitch * rb + 32 * ks);
        O.o[0][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[0], pb, O.o[0][rb], 0, 0, 0);
        O.o[1][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[1], pb, O.o[1][rb], 0, 0, 0);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// One token range of one request: Q load, pipelined tile loop, partial epilogue
// ------------------------------------------------------------------------------------

template <int FMT, bool PAGED>
__device__ __forceinline__ void run_range(const DecodeParams& p, uint8_t* bf0, uint8_t* bf1, uint8_t* st0,
                                          uint8_t* st1, const Shared& X, int b, int n, int rg, int lt0, int lt1,
                                          int64_t slot) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, lr = lane & 31, lh = lane >> 5;
  const int row0 = rg * kRowsPerGroup;                   // first row of this workgroup
  const int rows_here = min(kRowsPerGroup, p.rows - row0);
  const int nrb = (rows_here + 31) / 32;                 // row blocks with rows
  const int my_row = wave * kQkRows + (lane & 15);       // score-phase row (in the group)
  const bool active = wave * kQkRows < rows_here;        // this wavefront has score rows
  const int rc = min(row0 + my_row, p.rows - 1);

  ScoreState S;
  // rows past the end of the problem repeat the last row: finite values, never stored
  S.vis = max(n - p.q_len + rc / p.H + 1, 0);
  // fewest tokens any row of this wavefront sees: tiles below it need no mask
  int min_vis = S.vis;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) min_vis = min(min_vis, __shfl_xor(min_vis, o));
  S.m_used = -INFINITY;
  S.l_sum = 0.f;
  S.l_rnd = 0.f;
  {
    const uint16_t* qrow = p.q + ((int64_t)b * p.rows + rc) * kLatent;
    const uint16_t* prow = p.qpe + ((int64_t)b * p.rows + rc) * kRope;
#pragma unroll
    for (int k = 0; k < kQkSteps; ++k) {
      const int d = 32 * k + 8 * g;
      const uint16_t* src = (d < kLatent) ? qrow + d : prow + (d - kLatent);
      S.q[k] = *reinterpret_cast<const bf16x8*>(src);
    }
  }
  // chunk 4k + g of token t: (4k + g) ^ swz(t) = 8(k >> 1) + ((4(k & 1) + g) ^ swz(t)), and
  // swz(t + 16) = swz(t); byte offsets of whole 128-byte groups never have bit 6 set
  S.a_off = (lane & 15) * kTileRowBytes + ((g ^ swz(lane & 15)) << 4);
  S.p_off = my_row * kPRowPitch + 8 * g;

  OutState O;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) O.o[db][rb] = f32x16{};
  // transpose reads: in a group of 16 lanes (g, j = lane % 16), lane j addresses token
  // 16ks + 8(g >> 1) + 4e + j / 4 and dims d0 + 16(g & 1) + 4(j % 4) .. +4; lane i of
  // the group then receives dim d0 + 16(g & 1) + i of those four tokens.
  // (dims 32 apart are 4 chunks apart: chunk ^ 4 flips byte-offset bit 6; tokens 16
  // apart share the swizzle)
  {
    const int j = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tok = 8 * (g >> 1) + 4 * e + (j >> 2);
      const int dim = kPvDims * wave + 16 * (g & 1) + 4 * (j & 3);
      O.v_off[e] = tile_off(tok, dim >> 3) + 2 * (dim & 7);
    }
  }
  O.p_off = lr * kPRowPitch + 16 * lh;

  const float score_scale = p.score_scale;
  const int nt = lt1 - lt0;
  Range R{&p, b, n};

  // one tile: score phase, barrier, output phase (with `side` work issued inside it)
  auto tile_step = [&](const uint8_t* tile, int i, auto side) {
    const int tbase = (lt0 + i) * kTileTokens;
    score_tile(S, tile, X, tbase, score_scale, lane, active, active && tbase + kTileTokens <= min_vis, my_row);
    __syncthreads();
    out_tile(O, tile, X, nrb, lane, side);
  };
  auto nothing = [] {};

  if (nt > 0) {
    if (FMT == kFmtBf16) {
      // raw bf16 rows go straight into the two tiles; loads run one tile ahead
      load_bf16_tile<PAGED>(R, lt0 * kTileTokens, bf0, wave, lane);
      for (int i = 0;;) {
        wait_dma();
        __syncthreads();
        if (i + 1 < nt) load_bf16_tile<PAGED>(R, (lt0 + i + 1) * kTileTokens, bf1, wave, lane);
        tile_step(bf0, i, nothing);
        if (++i >= nt) break;
        wait_dma();
        __syncthreads();
        if (i + 1 < nt) load_bf16_tile<PAGED>(R, (lt0 + i + 1) * kTileTokens, bf0, wave, lane);
        tile_step(bf1, i, nothing);
        if (++i >= nt) break;
      }
    } else {
      // raw tiles are loaded two ahead of the MFMA work and dequantised one ahead, during
      // the output phase of the current tile (a dequantisation past the last tile only
      // rewrites an unused buffer)
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
        tile_step(bf0, i, [&] { dequant(st1, bf1); });
        if (++i >= nt) break;
        wait_dma();
        __syncthreads();
        if (i + 2 < nt) load_raw(i + 2, st1);
        tile_step(bf1, i, [&] { dequant(st0, bf0); });
        if (++i >= nt) break;
      }
    }
  }

  // ---- epilogue: the score-phase owner of each row publishes 1/l and writes lse ----
  {
    const float l_tot = quad_sum(S.l_sum);
    const float l_rnd = quad_sum(S.l_rnd);
    const bool ok = l_tot > 0.f;
    if (g == 0) {
      X.inv_l[my_row] = ok ? p.v_scale / l_rnd : 0.f;
      if (row0 + my_row < p.rows)
        p.lse_part[slot * p.l_slot + (int64_t)(row0 + my_row) * p.l_row] =
            ok ? (S.m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = row0 + 32 * rb + lr;
    if (rb < nrb && row < p.rows) {
      const float inv = X.inv_l[32 * rb + lr];
      float* orow = p.o_part + slot * p.o_slot + (int64_t)row * p.o_row + kPvDims * wave;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& o = O.o[db][rb];
          const f32x4 val = {o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * q4 + 4 * lh) = val;
        }
    }
  }
  __syncthreads();  // the next range reuses the LDS buffers
}

// ------------------------------------------------------------------------------------
// decode kernels
// ------------------------------------------------------------------------------------

// Contiguous: grid (row_groups, num_splits, B); split j covers [j*L, min((j+1)*L, S)).
__global__ __launch_bounds__(kThreads) void decode_contig_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t bf0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bf1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[kPBufBytes];
  __shared__ float alpha[kRowsPerGroup];
  __shared__ float inv_l[kRowsPerGroup];
  const Shared X{pbuf, alpha, inv_l};
  const int rg = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t0 = j * p.kv_len_per_split;
  const int t1 = min(t0 + p.kv_len_per_split, p.S);
  const int lt0 = t0 / kTileTokens;
  const int lt1 = (t1 + kTileTokens - 1) / kTileTokens;
  // slot b*H*NS + j with row = head addresses o_part [B, H, NS, 512]
  run_range<kFmtBf16, false>(p, bf0, bf1, nullptr, nullptr, X, b, p.S, rg, lt0, lt1,
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
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[kPBufBytes];
  __shared__ float alpha[kRowsPerGroup];
  __shared__ float inv_l[kRowsPerGroup];
  __shared__ int pre[kMaxBatch + 1];
  __shared__ int wsum[kWaves];
  const Shared X{pbuf, alpha, inv_l};
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
    run_range<FMT, true>(p, bf0, bf1, st0, st1, X, b, n, rg, t - pre[b], seg_end - pre[b], (int64_t)w + b);
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
