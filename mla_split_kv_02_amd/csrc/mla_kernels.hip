// gfx950 kernels for absorbed-MLA split-KV decode.
//
// Decode kernel.  One workgroup = 4 wavefronts, one per SIMD, so every wavefront has its
// SIMD's whole register file: its output accumulators (O^T, 512 dims x 32 rows, fp32 =
// 256 registers) live in the accumulation registers and its Q^T operand (32 rows x 576
// dims, 16-bit = 144 registers) in the vector registers.  The bf16 cache runs on bf16
// operands; the NVFP4 cache, dequantised exactly to f16, on f16 operands (the query row
// scaled by a power of two into f16, the weights in f16).  A workgroup owns up to 128 query
// rows (query x head) of one request and one token range; wavefront w owns rows
// 32w .. 32w+31 and does all of their arithmetic:
//   scores   S^T[32 tok x 32 rows] = K . Q^T         36 MFMA 32x32x16, K from LDS
//   softmax  online, base 2, lazy rescale; P^T is moved into the operand layout of the
//            output product with cross-half lane swaps, without touching LDS
//   output   O^T[512 x 32 rows] += V^T . P^T          32 MFMA 32x32x16, V^T read from the
//                                                      token-major tile with the LDS
//                                                      transpose read
// All heads of a request share one latent (absorbed MLA), so the four wavefronts work on
// the same LDS tile, which crosses HBM once per workgroup (the TileGym page's kernel
// re-reads it once per group of 16 heads).  The tile buffers are the only shared state:
// one workgroup barrier per tile hands them over.
//
// Per tile i (bf16, NVFP4): the global->LDS loads of a later tile are issued first; then
// the scores of tile i, with the softmax of tile i-1 (whose scores stayed in registers)
// spread between the score MFMAs, so the vector work issues while the matrix core is
// busy; then the output product of tile i-1, with NVFP4's dequantisation of tile i+1
// spread between its MFMAs in nine steps; then one barrier.  The first tile's softmax
// and the last tile's output product come after the loop.
//
// FP8 cache (run_range_fp8): 64-token tiles, none converted to bf16.  The bf16 query of
// each row is split exactly into two E4M3 operands (hi + lo, after a power-of-two row
// scale), so the scores run on FP8 MFMA 32x32x64 straight from the raw tile, each K
// operand read once for both terms (36 MFMAs per tile, two 32-token halves).  The softmax
// weights of each row and tile are scaled by a power of two 2^e that puts the tile's
// largest at 2^7..2^8 and split the same way (about 8 significant bits, like bf16), and
// the output product takes the raw tile's V^T through the 8-bit LDS transpose read: per
// 32 dims one V^T operand holding the tile's 64 tokens feeds two scaled MFMA 32x32x64,
// one with P_hi and one with P_lo, with the row's E8M0 scale 2^-e (32 MFMAs per tile).
// The matrix-core time per token is that of the bf16 path.
//
// Paged ranges are balanced by cost: a request costs its tiles plus a fixed overhead for
// its segment's query load, pipeline fill and partial store (decode_paged_kernel).
//
// FP8 query (cache format kFmtFp8Q, the TokenSpeed page's FP8 decode): the same loop
// with the query rounded to E4M3 once per range (72 registers) instead of split, so its
// scores take 18 FP8 MFMA 32x32x64 per 64-token tile instead of 36; the weights and the
// output product are those of the FP8 cache path.
//
// A sliding window (paged) starts each request's tiles at the one holding its first
// visible token and masks below the window; attention sinks enter in the combine.
//
// Combine kernels.  One wavefront per output row merges the partials with the split-K
// log-sum-exp reduce (TileGym page, forward: splitk_reduce), plus the row's sink logit
// when there is one.

#include "mla_internal.h"

#include <math.h>

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS uint8_t* lds_ptr;

constexpr int kKSteps = kRow / 16;                        // 36 K-steps of 16 dims (scores)
constexpr int kDimBlocks = kLatent / 32;                  // 16 output blocks of 32 dims
constexpr int kRowChunks = kRow * 2 / 16;                 // 72 bf16 chunks of 16 B per token
constexpr int kTileRowBytes = kRowChunks * 16;            // 1152
constexpr int kTileBytes = kTileTokens * kTileRowBytes;   // 36864
constexpr int kGroupBytes = kTileTokens * 128;            // 4096
constexpr int kBf16Loads = kTileBytes / 1024;             // 36 wavefront loads of 1 KiB
constexpr int kFp8RawBytes = kTileTokens * kRow;          // 18432
constexpr int kFp8Loads = kFp8RawBytes / 1024;            // 18
constexpr int kNvDataBytes = kRow / 2;                    // 288 packed E2M1 bytes per token
constexpr int kNvScaleBytes = kRow / 16;                  // 36 E4M3 scales per token
constexpr int kNvRawData = kTileTokens * kNvDataBytes;    // 9216
constexpr int kNvDataLoads = kNvRawData / 1024;           // 9
constexpr int kNvScaleWords = kTileTokens * kNvScaleBytes / 4;   // 288
constexpr int kNvScaleLoads = (kNvScaleWords + 63) / 64;          // 5 (the last one 32 words)
constexpr int kNvRawBytes = kNvRawData + 256 * kNvScaleLoads;     // 10496
constexpr float kTau = 8.0f;   // lazy rescale threshold (log2 units)
constexpr float kLn2 = 0.69314718055994531f;

// Buffers and load distance per cache format.  Tile i sits in 16-bit buffer i % kTiles
// (kStride bytes apart; bf16, or f16 dequantised from NVFP4); raw tile i (FP8 / NVFP4)
// in staging buffer i % kRaw.  In iteration i the loads of tile i + kAhead are issued.
// The FP8 formats (split loop) have no 16-bit tiles at all.
template <int FMT> struct Pipe;
template <> struct Pipe<kFmtBf16> {
  static constexpr int kTiles = 4, kStride = kTileBytes, kRaw = 0, kRawBytes = 0, kAhead = 2, kLoads = kBf16Loads;
};
template <> struct Pipe<kFmtNvfp4> {
  static constexpr int kTiles = 3, kStride = kTileBytes, kRaw = 3, kRawBytes = kNvRawBytes, kAhead = 3,
                       kLoads = kNvDataLoads + kNvScaleLoads;
};
// FP8 cache: raw 64-token tiles only (no bf16 copy); a tile is read by its score block
// and by the next iteration's output product, and the loads run two tiles ahead: four
// buffers of 36 KiB.
template <> struct Pipe<kFmtFp8> {
  static constexpr int kTiles = 0, kStride = 0, kRaw = 4, kRawBytes = 2 * kFp8RawBytes, kAhead = 2,
                       kLoads = kFp8Loads / 2;
};
// The FP8 query runs the same loop on the same raw tiles.
template <> struct Pipe<kFmtFp8Q> : Pipe<kFmtFp8> {};
template <int FMT> constexpr int smem_bytes() {
  return Pipe<FMT>::kTiles * Pipe<FMT>::kStride + Pipe<FMT>::kRaw * Pipe<FMT>::kRawBytes;
}
static_assert(smem_bytes<kFmtBf16>() <= 160 * 1024 && smem_bytes<kFmtFp8>() <= 160 * 1024 &&
                  smem_bytes<kFmtNvfp4>() <= 160 * 1024 && smem_bytes<kFmtFp8Q>() <= 160 * 1024,
              "LDS budget");

// Byte offset of 16-byte chunk c (0..71) of token row r in a 16-bit tile.  The tile is
// nine 4 KiB groups, one per 8 chunks (128 bytes) of every row: group c / 8 holds
// [32 rows][8 chunks], and inside a row the chunk position is XOR-swizzled with swz(r).
// Every global->LDS load instruction then fills one kilobyte of one group (8 rows), so
// each lane's source address is one per-tile base plus a multiple of 128 bytes.
// The swizzle keeps the three LDS access patterns free of bank conflicts (whether the
// LDS serves 16 or 32 lanes of a 16-byte access per cycle):
//   scores: rows 0..31 at one logical chunk  -> for any 8 rows of one parity within 16,
//           and for rows r, r + 4, .., r + 28, the positions differ;
//   output: transpose reads of rows t..t+3 and t+8..t+11 at chunks 0..3 -> rows two or
//           eight apart land in opposite halves of the 8-chunk group (position bit 2);
//   dequantisation writes: rows r, r+1 at all 8 chunks of a group.
// With u = (r / 2) % 8: position bit 2 = u0 ^ u2 ^ (r / 16) % 2, bits 1..0 = (u2, u1).
__device__ __forceinline__ int swz(int r) { return ((((r >> 1) ^ (r >> 3) ^ (r >> 4)) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int c) {
  return kGroupBytes * (c >> 3) + 128 * r + (((c & 7) ^ swz(r)) << 4);
}

// ------------------------------------------------------------------------------------
// Conversions
// ------------------------------------------------------------------------------------

__device__ __forceinline__ unsigned pack_hi16(float lo, float hi) {
  // bf16 pair from two floats whose low 16 bits are zero (exact conversion)
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// ------------------------------------------------------------------------------------
// Lane reductions
// ------------------------------------------------------------------------------------

// Values of lanes l and l ^ 32 combined with one cross-half lane swap (r[0] holds the low
// half's value in both halves, r[1] the high half's).
// max of three scores.  Scores are finite or -inf (masked), never NaN, so the operands need
// no quieting; written out because the compiler cannot know that of values produced by the
// score block and would quiet every operand first (one extra instruction each).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
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

// ------------------------------------------------------------------------------------
// Global -> LDS loads.  Each instruction runs on all 64 lanes and writes 16 (or 4) bytes
// per lane at LDS address lds + 16 * lane (4 * lane).  They are issued as inline assembly
// so that the compiler adds no waits of its own for them; every consumer waits with
// wait_vmcnt and a workgroup barrier.  The "s" forms take a wavefront-uniform 64-bit
// base and a per-lane 32-bit byte offset.
// ------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t lds_addr(lds_ptr p) { return (uint32_t)(uintptr_t)p; }
template <class T>
__device__ __forceinline__ LDS_AS T* at(uint32_t a) { return (LDS_AS T*)(uintptr_t)a; }

__device__ __forceinline__ void dma16_s(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
// dma16_s of base + OFF: the instruction's immediate offset moves the LDS destination by
// the same amount as the global source, so M0 takes lds - OFF.  Loads that share one base
// then need no 64-bit address arithmetic of their own.
template <int OFF>
__device__ __forceinline__ void dma16_o(const uint8_t* base, uint32_t voff, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(base), "i"(OFF), "{m0}"(lds - OFF)
               : "memory");
}
__device__ __forceinline__ void dma4_s(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Wait until at most n of this wavefront's vector-memory operations are outstanding
// (they complete in issue order).  n is wavefront-uniform.
__device__ __forceinline__ void wait_vmcnt(int n) {
#define MLA_VMCNT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
  switch (n) {
    MLA_VMCNT_CASE(1) MLA_VMCNT_CASE(2) MLA_VMCNT_CASE(3) MLA_VMCNT_CASE(4) MLA_VMCNT_CASE(5)
    MLA_VMCNT_CASE(6) MLA_VMCNT_CASE(7) MLA_VMCNT_CASE(8) MLA_VMCNT_CASE(9) MLA_VMCNT_CASE(10)
    MLA_VMCNT_CASE(11) MLA_VMCNT_CASE(12) MLA_VMCNT_CASE(13) MLA_VMCNT_CASE(14) MLA_VMCNT_CASE(15)
    MLA_VMCNT_CASE(16) MLA_VMCNT_CASE(17) MLA_VMCNT_CASE(18)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
#undef MLA_VMCNT_CASE
}

// ------------------------------------------------------------------------------------
// Tile sources.  Tokens past the end of the request are clamped to its last token
// (their scores are masked, and a real row keeps every value finite); a 32-token tile
// never crosses a page (page sizes 32 and 64), so one block-table entry serves a tile.
// Load instruction j of a tile is issued by wavefront j % 4, as its (j / 4)-th; every
// lane keeps one source row for the whole tile, and its source address moves by a
// fixed stride from one of its instructions to the next (added to the uniform base).
// ------------------------------------------------------------------------------------

struct Src {
  const DecodeParams* p;
  int b;  // request
  int n;  // its tokens (>= 1 whenever a tile is loaded)
};

// Block-table entry of tile tb.  The table is only read by the kernel, so it is read
// through the constant address space: a scalar load, whose wait the compiler places
// at the first use.  The kernel reads the entry one tile before the loads that use it,
// which keeps the load latency off the critical path (a vector load here would be
// waited for together with the tile loads in flight).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int table_entry(const Src& S, int tb) {
  const DecodeParams& p = *S.p;
  return ((const_i32_ptr)p.block_tables)[(int64_t)S.b * p.max_blocks + (tb >> p.page_shift)];
}
// Start of the page an entry names, clamped into the cache.
__device__ __forceinline__ const uint8_t* page_start(const Src& S, int entry) {
  const DecodeParams& p = *S.p;
  return p.cache + (int64_t)min(max(entry, 0), p.num_pages - 1) * p.page_stride;
}

// bf16 rows straight into the tile.  Instruction j = 4m + w fills group m, rows 8w ..
// 8w+7: lane l takes row 8w + l/8 and the chunk whose swizzled position is l % 8.
template <bool PAGED>
__device__ __forceinline__ void load_bf16_tile(const Src& S, int tb, const uint8_t* pg, uint32_t tile, int wave,
                                               int lane) {
  const DecodeParams& p = *S.p;
  const int r = 8 * wave + (lane >> 3);
  const int tok = min(tb + r, S.n - 1);
  const int cpos = ((lane & 7) ^ swz(r)) << 4;  // byte offset of the chunk inside its group of 8
  const uint32_t lds = tile + 1024 * wave;
  if (PAGED) {
    const int rip = tb & (p.page_size - 1);
    const uint32_t voff = (uint32_t)((rip + tok - tb) * (2 * kRow) + cpos);
    dma16_o<0>(pg, voff, lds);
    dma16_o<128>(pg, voff, lds + kGroupBytes);
    dma16_o<256>(pg, voff, lds + kGroupBytes * 2);
    dma16_o<384>(pg, voff, lds + kGroupBytes * 3);
    dma16_o<512>(pg, voff, lds + kGroupBytes * 4);
    dma16_o<640>(pg, voff, lds + kGroupBytes * 5);
    dma16_o<768>(pg, voff, lds + kGroupBytes * 6);
    dma16_o<896>(pg, voff, lds + kGroupBytes * 7);
    dma16_o<1024>(pg, voff, lds + kGroupBytes * 8);
  } else {
    const int64_t t0 = (int64_t)S.b * p.S + tb;
    const uint8_t* kv = reinterpret_cast<const uint8_t*>(p.kv + t0 * kLatent);
    const uint8_t* kpe = reinterpret_cast<const uint8_t*>(p.kpe + t0 * kRope);
    const uint32_t kvoff = (uint32_t)((tok - tb) * (2 * kLatent) + cpos);
    dma16_o<0>(kv, kvoff, lds);
    dma16_o<128>(kv, kvoff, lds + kGroupBytes);
    dma16_o<256>(kv, kvoff, lds + kGroupBytes * 2);
    dma16_o<384>(kv, kvoff, lds + kGroupBytes * 3);
    dma16_o<512>(kv, kvoff, lds + kGroupBytes * 4);
    dma16_o<640>(kv, kvoff, lds + kGroupBytes * 5);
    dma16_o<768>(kv, kvoff, lds + kGroupBytes * 6);
    dma16_o<896>(kv, kvoff, lds + kGroupBytes * 7);
    dma16_s(kpe, (uint32_t)((tok - tb) * (2 * kRope) + cpos), lds + kGroupBytes * 8);
  }
}

// FP8 rows, raw.  Staging layout: chunk c (16 codes) of row r at 2048 (c / 4) + 64 r +
// 16 p, p = (c % 4) ^ sswz(r).  Instruction j = 4m + w covers chunk group j / 2 of rows
// 16 (j % 2) ..: lane l takes row 16 (w % 2) + l / 4 and the chunk 4 (w / 2 + 2m) + c % 4
// that belongs at position l % 4.
// The swizzle: row bits 2 and 3 flip position bits 0 and 1 (and row bit 4 position bit 0
// again).  A row is 64 bytes, so the bank of (row r, position p) depends on r % 4 and p.
// The score reads (16 lanes per cycle: rows r .. r+15 at one logical chunk) are
// conflict-free: the four rows of each residue mod 4 take four different positions.  So
// are the 8-bit transpose reads of the 64-token loop (32 lanes per cycle: tokens
// b + {0..3, 8..11} with b % 16 in {0, 4}, two adjacent chunks, two 8-byte halves): the
// tokens j and j + 8 of one residue differ in position bit 1 and the two chunks in bit 0.
__device__ __forceinline__ int sswz(int r) { return ((r >> 2) & 3) ^ ((r >> 4) & 1); }

__device__ __forceinline__ void load_fp8_raw(const Src& S, int tb, const uint8_t* pg, uint32_t st, int wave, int lane) {
  const int rip = tb & (S.p->page_size - 1);
  const int r = 16 * (wave & 1) + (lane >> 2);
  const int tok = min(tb + r, S.n - 1);
  const int c4 = (lane & 3) ^ sswz(r);
  const uint32_t voff = (uint32_t)((rip + tok - tb) * kRow + 16 * (4 * (wave >> 1) + c4));
  // 18 instructions: four from every wavefront, a fifth from wavefronts 0 and 1 (a
  // wavefront-uniform branch, so the condition stays in scalar registers)
  static_assert(kFp8Loads > 16 && kFp8Loads <= 20, "four or five loads per wavefront");
  dma16_o<0>(pg, voff, st + 1024 * wave);
  dma16_o<128>(pg, voff, st + 1024 * (4 + wave));
  dma16_o<256>(pg, voff, st + 1024 * (8 + wave));
  dma16_o<384>(pg, voff, st + 1024 * (12 + wave));
  if (wave < kFp8Loads - 16) dma16_o<512>(pg, voff, st + 1024 * (16 + wave));
}

// NVFP4 rows, raw.  Data: chunk c (32 codes) of row r at 1024 (c / 2) + 32 r + 16 (c % 2);
// instruction j < 9 covers chunks 2j, 2j+1 of all rows (lane l: row l / 2, chunk
// 2j + l % 2).  Scales: instruction 9 + s writes 256 bytes at 9216 + 256 s, lane l the
// dword min(2s + l % 2, 8) of row l / 2 (the repeated dword 8 lands in a spare slot).
__device__ __forceinline__ void load_nvfp4_raw(const Src& S, int tb, const uint8_t* pg, uint32_t st, int wave,
                                               int lane) {
  const DecodeParams& p = *S.p;
  const int rip = tb & (p.page_size - 1);
  const int r = lane >> 1;
  const int tok = min(tb + r, S.n - 1);
  const int prow = rip + tok - tb;
  const uint32_t dvoff = (uint32_t)(prow * kNvDataBytes + 16 * (lane & 1));
  auto scales = [&](int sidx) {  // scale instruction sidx (0..4)
    const int q = min(2 * sidx + (lane & 1), kNvScaleBytes / 4 - 1);
    dma4_s(pg, (uint32_t)(p.page_size * kNvDataBytes + prow * kNvScaleBytes + 4 * q), st + kNvRawData + 256 * sidx);
  };
  // instruction j = 4m + wave as above, with wavefront-uniform branches (so the conditions
  // stay in scalar registers): m = 0, 1 data; m = 2 data 8 (wavefront 0) or scales 0..2;
  // m = 3 scales 3, 4 (wavefronts 0, 1)
  static_assert(kNvDataLoads == 9 && kNvScaleLoads == 5, "load split below");
  dma16_o<0>(pg + 32 * wave, dvoff, st + 1024 * wave);
  dma16_o<128>(pg + 32 * wave, dvoff, st + 1024 * (4 + wave));
  if (wave == 0) dma16_o<256>(pg, dvoff, st + 1024 * 8);
  else scales(wave - 1);
  if (wave < 2) scales(3 + wave);
}

// Raw NVFP4 staging -> f16 tile.  Thread t writes chunk t % 8 of group m of row t / 8:
// eight codes (4 data bytes at 1024 m + 32 r + 4 (t % 8)) times their scale (group
// (t % 8) / 2 + 4m of the row: byte (t % 8) / 2 of scale dword m).  With the scale
// s = 2^E M (M in [1, 2), signed), the scaled FP4 conversion gives code x 2^E (it takes
// only the exponent of its scale operand) as packed f16, and one packed f16 multiply by
// M finishes the product.  Every product has at most 6 significant bits and lies in
// [2^-10, 1536] (or is 0), so each step is exact in f16; a NaN scale gives NaN.
// The work is cut into nine steps, one per 4 KiB group m of the f16 tile, so that the
// output phase can spread them between its MFMAs: read(m) fetches the step's code dword
// and scale byte, put(m) converts and writes them.
struct NvDequant {
  uint32_t rd, sd, wr;
  unsigned w[9];
  unsigned char sc[9];
  __device__ __forceinline__ NvDequant(uint32_t st, uint32_t tile, int tid) {
    const int r = tid >> 3, t7 = tid & 7;
    rd = st + 32 * r + 4 * t7;                   // + 1024 m
    sd = st + kNvRawData + 8 * r + (t7 >> 1);    // + 256 (m/2) + 4 (m%2)
    wr = tile + 128 * r + ((t7 ^ swz(r)) << 4);  // + 4096 m
  }
  __device__ __forceinline__ void read(int m) {
    w[m] = *at<unsigned>(rd + 1024 * m);
    sc[m] = *at<unsigned char>(sd + 256 * (m >> 1) + 4 * (m & 1));
  }
  __device__ __forceinline__ void put(int m) {
    const float scale = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc[m], false)[0];
    const float mant = __uint_as_float((__float_as_uint(scale) & 0x807FFFFFu) | 0x3F800000u);  // +-M
    const f16x2 m2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(mant, mant));  // exact: 4 bits
    const f16x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[m], scale, 0) * m2;
    const f16x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[m], scale, 1) * m2;
    const f16x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[m], scale, 2) * m2;
    const f16x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[m], scale, 3) * m2;
    *at<u32x4>(wr + kGroupBytes * m) =
        u32x4{__builtin_bit_cast(unsigned, f0), __builtin_bit_cast(unsigned, f1), __builtin_bit_cast(unsigned, f2),
              __builtin_bit_cast(unsigned, f3)};
  }
};

__device__ __forceinline__ void dequant_nvfp4(uint32_t st, uint32_t tile, int tid) {
  NvDequant d(st, tile, tid);
#pragma unroll
  for (int m = 0; m < 9; ++m) d.read(m);
#pragma unroll
  for (int m = 0; m < 9; ++m) d.put(m);
}

// ------------------------------------------------------------------------------------
// Per-wavefront arithmetic.  MFMA 32x32x16 bf16 operand layouts (lane l, element e):
// A[i = l % 32][k = 8 (l / 32) + e], B[k = 8 (l / 32) + e][j = l % 32]; result register v
// of lane l holds D[i = 8 (v / 4) + 4 (l / 32) + v % 4][j = l % 32].
// ------------------------------------------------------------------------------------

// The instruction block of qk_tile, for MF the MFMA 32x32x16 on bf16 or on f16 operands.
#define MLA_QK_TILE_ASM(MF) \
  asm volatile( \
  "ds_read_b128 %[a0], %[b0] offset:0\n\t" \
  "ds_read_b128 %[a1], %[b1] offset:0\n\t" \
  "ds_read_b128 %[a2], %[b2] offset:0\n\t" \
  "ds_read_b128 %[a3], %[b3] offset:0\n\t" \
  "ds_read_b128 %[a4], %[b0] offset:4096\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q0], 0\n\t" \
  "ds_read_b128 %[a5], %[b1] offset:4096\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q1], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b2] offset:4096\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q2], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b3] offset:4096\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q3], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b0] offset:8192\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q4], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b1] offset:8192\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q5], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b2] offset:8192\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q6], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b3] offset:8192\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q7], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b0] offset:12288\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q8], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b1] offset:12288\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q9], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b2] offset:12288\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q10], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b3] offset:12288\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q11], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b0] offset:16384\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q12], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b1] offset:16384\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q13], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b2] offset:16384\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q14], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b3] offset:16384\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q15], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b0] offset:20480\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q16], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b1] offset:20480\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q17], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b2] offset:20480\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q18], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b3] offset:20480\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q19], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b0] offset:24576\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q20], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b1] offset:24576\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q21], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b2] offset:24576\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q22], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b3] offset:24576\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q23], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b0] offset:28672\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q24], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b1] offset:28672\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q25], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b2] offset:28672\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q26], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b3] offset:28672\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q27], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b0] offset:32768\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q28], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b1] offset:32768\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q29], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b2] offset:32768\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q30], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b3] offset:32768\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q31], %[s]\n\t" \
  "s_waitcnt lgkmcnt(3)\n\t" \
  MF " %[s], %[a4], %[q32], %[s]\n\t" \
  "s_waitcnt lgkmcnt(2)\n\t" \
  MF " %[s], %[a5], %[q33], %[s]\n\t" \
  "s_waitcnt lgkmcnt(1)\n\t" \
  MF " %[s], %[a6], %[q34], %[s]\n\t" \
  "s_waitcnt lgkmcnt(0)\n\t" \
  MF " %[s], %[a0], %[q35], %[s]\n\t" \
  "s_nop 7\n\ts_nop 7\n\ts_nop 7" \
  : [s] "=&v"(s), [a0] "=&v"(a0), [a1] "=&v"(a1), [a2] "=&v"(a2), [a3] "=&v"(a3), [a4] "=&v"(a4), [a5] "=&v"(a5), [a6] "=&v"(a6) \
  : [b0] "v"(b0), [b1] "v"(b1), [b2] "v"(b2), [b3] "v"(b3), \
  [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]), \
  [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]), \
  [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]), \
  [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]), \
  [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]), \
  [q30] "v"(q[30]), [q31] "v"(q[31]), [q32] "v"(q[32]), [q33] "v"(q[33]), [q34] "v"(q[34]), [q35] "v"(q[35]) \
  : "memory")

// Scores of one tile: S^T[token][row], A = K (token l % 32, dims 16k + 8 (l / 32) ..),
// B = Q^T (in registers).  K-step k reads chunk 2k + l/32 of the lane's token row: group
// k / 4, swizzled position 2 (k % 4) + l/32, i.e. address ab[k % 4] + 4096 (k / 4) past
// the tile.  The accumulation registers all hold the output, so this chain accumulates
// in vector registers, which the compiler does not give MFMA results; it is written out
// as one instruction block: operand reads run five K-steps ahead (about the LDS read
// latency over the MFMA issue interval) through seven operand buffers, each MFMA waits
// only for its own operand (LDS reads complete in order), and
// back-to-back MFMAs accumulating into the same registers need no wait states.  The
// closing s_nop run gives the wait states (more than the 18 required) before vector ALU
// instructions may read the result.
template <bool H = false>
__device__ __forceinline__ f32x16 qk_tile(const bf16x8* q, uint32_t tile, const int* ab) {
  const uint32_t b0 = tile + ab[0], b1 = tile + ab[1], b2 = tile + ab[2], b3 = tile + ab[3];
  f32x16 s;
  bf16x8 a0, a1, a2, a3, a4, a5, a6;
  if constexpr (H)
    MLA_QK_TILE_ASM("v_mfma_f32_32x32x16_f16");
  else
    MLA_QK_TILE_ASM("v_mfma_f32_32x32x16_bf16");
  return s;
}


// Output product of one tile: O^T[dim][row] += V^T[dim][token] . P^T[token][row] for the
// 16 blocks of 32 dims and the two K-steps of 16 tokens.  V^T comes from two transpose
// reads per operand (vb[2e]: tokens 4e .. of the lane's half.  Dims 32 apart are 4
// chunks apart, i.e. position bit 2 (byte-offset bit 6) flipped inside the same group;
// 64 dims apart are one group further; tokens 16 apart have position bit 2 of the
// swizzle flipped, so the second K-step flips byte-offset bit 6 as well; vb[2e + 1] is
// vb[2e] with that bit flipped).  pp holds P^T.  NB blocks from block db0 (even) into
// o[0 .. NB): the wavefront's share of the 512 dims when several share one row block.
// c += a . b on the 32x32x16 matrix core, operands bf16 or (H) f16, held as 16-byte vectors
template <bool H>
__device__ __forceinline__ f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (H)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int NB = kDimBlocks, bool H = false>
__device__ __forceinline__ void pv_tile(f32x16* o, uint32_t tile, const unsigned* pp, const int* vb, int db0 = 0) {
  uint32_t base[4];  // [e][db & 1]
#pragma unroll
  for (int x = 0; x < 4; ++x) base[x] = tile + vb[x] + kGroupBytes * (db0 >> 1);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]});
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const uint32_t off = kGroupBytes * (db >> 1) + 16 * 128 * ks;
      const int flip = (db & 1) ^ ks;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at<s16x4>(base[flip] + off));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at<s16x4>(base[2 + flip] + off));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = mfma16<H>(va, pb, o[db]);
    }
  }
}

// Wait states before the accumulators may be read after an MFMA issued as an assembly
// statement (the FP8 split path's output product), which the compiler cannot see.
__device__ __forceinline__ void mfma_drain_any() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// o *= alpha in place in the accumulation registers (NB blocks), one value at a time
// through one vector register.
template <int NB = kDimBlocks>
__device__ __forceinline__ void rescale(f32x16* o, float alpha) {
  mfma_drain_any();
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float e = o[db][v], t;
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                   : "+a"(e), "=&v"(t)
                   : "v"(alpha));
      o[db][v] = e;
    }
}

// e * f for an accumulator e, read from its accumulation register into a vector
// register without writing it back (the compiler would otherwise stage all of them).
__device__ __forceinline__ float scaled(float e, float f) {
  float t;
  asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2" : "=&v"(t) : "a"(e), "v"(f));
  return t;
}

struct Softmax {
  float m_used;  // reference max of the row (log2 domain), equal in lanes l and l ^ 32
  float l_sum;   // this lane's share of sum p (unrounded): for the LSE
  float l_rnd;   // this lane's share of sum bf16(p): normalises O
};

// Online softmax of one tile.  x: raw scores of this lane (row l % 32, tokens
// 8 (v / 4) + 4 (l / 32) + v % 4), masked ones already -inf; c > 0 is the score scale in
// log2 units.  Returns the factor for the row's accumulators before this tile's
// product and P^T in the output product's B layout: pp[4 ks + ..] holds tokens
// 16 ks + 8 (l / 32) .. + 8 of the row.
template <bool H = false>
__device__ __forceinline__ float softmax_tile(Softmax& S, float* x, float c, unsigned* pp) {
  float mt = x[0];
#pragma unroll
  for (int v = 1; v < 15; v += 2) mt = max3(mt, x[v], x[v + 1]);
  mt = max3(mt, x[15], x[15]);
  mt = pair_max(mt) * c;  // -inf stays -inf (c > 0)
  const bool need = mt > S.m_used + kTau;
  const float m_new = need ? mt : S.m_used;
  // (while no token has been seen the accumulators are zero and need no factor)
  const float alpha = (need && S.m_used != -INFINITY) ? __builtin_amdgcn_exp2f(S.m_used - m_new) : 1.0f;
  S.l_sum *= alpha;
  S.l_rnd *= alpha;
  S.m_used = m_new;
  const float nm = (m_new == -INFINITY) ? 0.f : -m_new;
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = __builtin_amdgcn_exp2f(fmaf(x[v], c, nm));
  float acc = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc += e[v];
  S.l_sum += acc;
  unsigned d[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    if constexpr (H) {
      const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      const f16x2 pr = {(_Float16)e[2 * v], (_Float16)e[2 * v + 1]};
      S.l_rnd = __builtin_amdgcn_fdot2(pr, ones, S.l_rnd, false);
      d[v] = __builtin_bit_cast(unsigned, pr);
    } else {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      const bf16x2 pr = {(__bf16)e[2 * v], (__bf16)e[2 * v + 1]};
      S.l_rnd = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, S.l_rnd, false);
      d[v] = __builtin_bit_cast(unsigned, pr);
    }
  }
  // d[4ks + 0..1]: tokens 16ks + 4 (l/32) + 0..3; d[4ks + 2..3]: tokens 16ks + 8 + 4 (l/32) + 0..3.
  // The low half needs tokens 16ks + 0..7 (its own d0 d1, then the high half's d0 d1), the
  // high half tokens 16ks + 8..15 (the low half's d2 d3, then its own d2 d3).
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const auto r02 = __builtin_amdgcn_permlane32_swap(d[4 * ks + 0], d[4 * ks + 2], false, false);
    const auto r13 = __builtin_amdgcn_permlane32_swap(d[4 * ks + 1], d[4 * ks + 3], false, false);
    pp[4 * ks + 0] = r02[0];
    pp[4 * ks + 1] = r13[0];
    pp[4 * ks + 2] = r02[1];
    pp[4 * ks + 3] = r13[1];
  }
  return alpha;
}

// The instruction block of qk_softmax_tile, for bf16 or f16 operands: MF the MFMA
// 32x32x16, CV the packing conversion of the weights, DT the dot product that adds a
// packed pair of rounded weights to l_rnd (its second operand the pair (1, 1)).
#define MLA_QK_SOFTMAX_ASM(MF, CV, DT) \
  asm volatile( \
  "ds_read_b128 %[a0], %[b0] offset:0\n\t" \
  "ds_read_b128 %[a1], %[b1] offset:0\n\t" \
  "ds_read_b128 %[a2], %[b2] offset:0\n\t" \
  "ds_read_b128 %[a3], %[b3] offset:0\n\t" \
  "ds_read_b128 %[a4], %[b0] offset:4096\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q0], 0\n\t" \
  "ds_read_b128 %[a5], %[b1] offset:4096\n\t" \
  "v_max3_f32 %[t0], %[x0], %[x1], %[x2]\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x3], %[x4]\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x5], %[x6]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q1], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b2] offset:4096\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x7], %[x8]\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x9], %[x10]\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x11], %[x12]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q2], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b3] offset:4096\n\t" \
  "v_max3_f32 %[t0], %[t0], %[x13], %[x14]\n\t" \
  "v_max_f32 %[t0], %[t0], %[x15]\n\t" \
  "v_mov_b32 %[t1], %[t0]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q3], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b0] offset:8192\n\t" \
  "v_permlane32_swap_b32 %[t0], %[t1]\n\t" \
  "v_max_f32 %[t0], %[t0], %[t1]\n\t" \
  "v_mul_f32 %[t0], %[c], %[t0]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q4], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b1] offset:8192\n\t" \
  "v_add_f32 %[t1], 0x41000000, %[m]\n\t" \
  "v_cmp_gt_f32 vcc, %[t0], %[t1]\n\t" \
  "v_cndmask_b32 %[t1], %[m], %[t0], vcc\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q5], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b2] offset:8192\n\t" \
  "v_sub_f32 %[t2], %[m], %[t1]\n\t" \
  "v_exp_f32 %[t2], %[t2]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q6], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b3] offset:8192\n\t" \
  "v_cndmask_b32 %[al], 1.0, %[t2], vcc\n\t" \
  "v_cmp_eq_f32 vcc, 0xff800000, %[m]\n\t" \
  "v_cndmask_b32_e64 %[al], %[al], 1.0, vcc\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q7], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b0] offset:12288\n\t" \
  "v_mul_f32 %[ls], %[ls], %[al]\n\t" \
  "v_mul_f32 %[lr], %[lr], %[al]\n\t" \
  "v_mov_b32 %[m], %[t1]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q8], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b1] offset:12288\n\t" \
  "v_cmp_eq_f32 vcc, 0xff800000, %[t1]\n\t" \
  "v_cndmask_b32_e64 %[t2], -%[t1], 0, vcc\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q9], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b2] offset:12288\n\t" \
  "v_fma_f32 %[x0], %[x0], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x0], %[x0]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q10], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b3] offset:12288\n\t" \
  "v_fma_f32 %[x1], %[x1], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x1], %[x1]\n\t" \
  "v_add_f32 %[t0], 0, %[x0]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q11], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b0] offset:16384\n\t" \
  "v_fma_f32 %[x2], %[x2], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x2], %[x2]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x1]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q12], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b1] offset:16384\n\t" \
  "v_fma_f32 %[x3], %[x3], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x3], %[x3]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x2]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q13], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b2] offset:16384\n\t" \
  "v_fma_f32 %[x4], %[x4], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x4], %[x4]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x3]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q14], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b3] offset:16384\n\t" \
  "v_fma_f32 %[x5], %[x5], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x5], %[x5]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x4]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q15], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b0] offset:20480\n\t" \
  "v_fma_f32 %[x6], %[x6], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x6], %[x6]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x5]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q16], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b1] offset:20480\n\t" \
  "v_fma_f32 %[x7], %[x7], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x7], %[x7]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x6]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q17], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b2] offset:20480\n\t" \
  "v_fma_f32 %[x8], %[x8], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x8], %[x8]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x7]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q18], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b3] offset:20480\n\t" \
  "v_fma_f32 %[x9], %[x9], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x9], %[x9]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x8]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q19], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b0] offset:24576\n\t" \
  "v_fma_f32 %[x10], %[x10], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x10], %[x10]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x9]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q20], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b1] offset:24576\n\t" \
  "v_fma_f32 %[x11], %[x11], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x11], %[x11]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x10]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q21], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b2] offset:24576\n\t" \
  "v_fma_f32 %[x12], %[x12], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x12], %[x12]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x11]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q22], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b3] offset:24576\n\t" \
  "v_fma_f32 %[x13], %[x13], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x13], %[x13]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x12]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q23], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b0] offset:28672\n\t" \
  "v_fma_f32 %[x14], %[x14], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x14], %[x14]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x13]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q24], %[s]\n\t" \
  "ds_read_b128 %[a1], %[b1] offset:28672\n\t" \
  "v_fma_f32 %[x15], %[x15], %[c], %[t2]\n\t" \
  "v_exp_f32 %[x15], %[x15]\n\t" \
  "v_add_f32 %[t0], %[t0], %[x14]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a4], %[q25], %[s]\n\t" \
  "ds_read_b128 %[a2], %[b2] offset:28672\n\t" \
  "v_add_f32 %[t0], %[t0], %[x15]\n\t" \
  "v_add_f32 %[ls], %[ls], %[t0]\n\t" \
  CV " %[x0], %[x0], %[x1]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a5], %[q26], %[s]\n\t" \
  "ds_read_b128 %[a3], %[b3] offset:28672\n\t" \
  DT " %[x0]\n\t" \
  CV " %[x1], %[x2], %[x3]\n\t" \
  DT " %[x1]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a6], %[q27], %[s]\n\t" \
  "ds_read_b128 %[a4], %[b0] offset:32768\n\t" \
  CV " %[x2], %[x4], %[x5]\n\t" \
  DT " %[x2]\n\t" \
  CV " %[x3], %[x6], %[x7]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a0], %[q28], %[s]\n\t" \
  "ds_read_b128 %[a5], %[b1] offset:32768\n\t" \
  DT " %[x3]\n\t" \
  CV " %[x4], %[x8], %[x9]\n\t" \
  DT " %[x4]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a1], %[q29], %[s]\n\t" \
  "ds_read_b128 %[a6], %[b2] offset:32768\n\t" \
  CV " %[x5], %[x10], %[x11]\n\t" \
  DT " %[x5]\n\t" \
  CV " %[x6], %[x12], %[x13]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a2], %[q30], %[s]\n\t" \
  "ds_read_b128 %[a0], %[b3] offset:32768\n\t" \
  DT " %[x6]\n\t" \
  CV " %[x7], %[x14], %[x15]\n\t" \
  DT " %[x7]\n\t" \
  "s_waitcnt lgkmcnt(4)\n\t" \
  MF " %[s], %[a3], %[q31], %[s]\n\t" \
  "v_permlane32_swap_b32 %[x0], %[x2]\n\t" \
  "v_permlane32_swap_b32 %[x1], %[x3]\n\t" \
  "s_waitcnt lgkmcnt(3)\n\t" \
  MF " %[s], %[a4], %[q32], %[s]\n\t" \
  "v_permlane32_swap_b32 %[x4], %[x6]\n\t" \
  "v_permlane32_swap_b32 %[x5], %[x7]\n\t" \
  "s_waitcnt lgkmcnt(2)\n\t" \
  MF " %[s], %[a5], %[q33], %[s]\n\t" \
  "s_waitcnt lgkmcnt(1)\n\t" \
  MF " %[s], %[a6], %[q34], %[s]\n\t" \
  "s_waitcnt lgkmcnt(0)\n\t" \
  MF " %[s], %[a0], %[q35], %[s]\n\t" \
  "s_nop 7\n\ts_nop 7\n\ts_nop 7" \
  : [s] "=&v"(s), [a0] "=&v"(a0), [a1] "=&v"(a1), [a2] "=&v"(a2), [a3] "=&v"(a3), [a4] "=&v"(a4), [a5] "=&v"(a5), \
  [a6] "=&v"(a6), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [al] "=&v"(alpha), [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), \
  [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]), [x8] "+v"(x[8]), \
  [x9] "+v"(x[9]), [x10] "+v"(x[10]), [x11] "+v"(x[11]), [x12] "+v"(x[12]), [x13] "+v"(x[13]), \
  [x14] "+v"(x[14]), [x15] "+v"(x[15]), [m] "+v"(S.m_used), [ls] "+v"(S.l_sum), [lr] "+v"(S.l_rnd) \
  : [b0] "v"(b0), [b1] "v"(b1), [b2] "v"(b2), [b3] "v"(b3), [c] "v"(c), \
  [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]), \
  [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]), \
  [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]), \
  [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]), \
  [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]), \
  [q30] "v"(q[30]), [q31] "v"(q[31]), [q32] "v"(q[32]), [q33] "v"(q[33]), [q34] "v"(q[34]), [q35] "v"(q[35]) \
  : "vcc", "memory")

// Scores of tile i as in qk_tile, with the online softmax of tile i-1 (the same steps
// as softmax_tile) spread over the MFMA chain: vector ALU work on registers the chain
// does not touch, which issues while the matrix core is busy.  x: the raw scores of
// tile i-1 (masked), used up (P^T is formed in x[0..7]); S: the row state; pp: P^T of
// tile i-1 in the output product's B layout; alpha: the factor for the accumulators before
// that tile's product.  Hazards are covered by the instruction order: a transcendental
// result is read three or more instructions later, a cross-half swap reads registers
// written two or more instructions earlier, and vcc is written and read only by these
// steps.
template <bool H = false>
__device__ __forceinline__ f32x16 qk_softmax_tile(const bf16x8* q, uint32_t tile, const int* ab, float* x,
                                                  Softmax& S, float c, unsigned* pp, float& alpha) {
  const uint32_t b0 = tile + ab[0], b1 = tile + ab[1], b2 = tile + ab[2], b3 = tile + ab[3];
  f32x16 s;
  bf16x8 a0, a1, a2, a3, a4, a5, a6;
  float t0, t1, t2;
  if constexpr (H)
    MLA_QK_SOFTMAX_ASM("v_mfma_f32_32x32x16_f16", "v_cvt_pk_f16_f32", "v_dot2c_f32_f16 %[lr], 0x3c003c00,");
  else
    MLA_QK_SOFTMAX_ASM("v_mfma_f32_32x32x16_bf16", "v_cvt_pk_bf16_f32", "v_dot2c_f32_bf16 %[lr], 0x3f803f80,");
#pragma unroll
  for (int j = 0; j < 8; ++j) pp[j] = __float_as_uint(x[j]);  // P^T went into x[0..7]
  return s;
}

// Output product of tile i-1 (vtile, P^T in pp): 2 NB MFMAs (NB dim blocks from block
// db0, even), V^T from the transpose reads four MFMAs ahead (bf16 and NVFP4 caches; the
// softmax ran in the score block).  nv: the NVFP4 dequantisation of the next tile, spread
// over the MFMAs (step m after MFMA 3m + 2, its reads two steps earlier); null for the
// other formats, and only with all 16 blocks.
template <int NB = kDimBlocks, bool H = false>
__device__ __forceinline__ void output_phase(f32x16* o, uint32_t vtile, const unsigned* pp, const int* vb,
                                             NvDequant* nv = nullptr, int db0 = 0) {
  constexpr int kAhead = 4;
  uint32_t base[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) base[v] = vtile + vb[v] + kGroupBytes * (db0 >> 1);
  const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pp[0], pp[1], pp[2], pp[3]});
  const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pp[4], pp[5], pp[6], pp[7]});
  auto tr = [&](int k) {  // V^T operand of output MFMA k (dims block k % NB, K-step k / NB)
    const int db = k % NB, ks = k / NB, flip = (db & 1) ^ ks;
    const uint32_t off = kGroupBytes * (db >> 1) + 16 * 128 * ks;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at<s16x4>(base[flip] + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at<s16x4>(base[2 + flip] + off));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 va[2 * NB];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) va[k] = tr(k);
  if (NB == kDimBlocks && nv) {
    nv->read(0);
    nv->read(1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 2 * NB; ++k) {
    o[k % NB] = mfma16<H>(va[k], (k < NB) ? pb0 : pb1, o[k % NB]);
    if (k + kAhead < 2 * NB) va[k + kAhead] = tr(k + kAhead);
    if (NB == kDimBlocks && nv && k % 3 == 2 && k / 3 < 9) {
      nv->put(k / 3);
      if (k / 3 + 2 < 9) nv->read(k / 3 + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------------------------
// FP8 cache: the split path.  The FP8 matrix core multiplies E4M3 codes exactly and
// accumulates in fp32, so a bf16 operand can ride on it as two E4M3 operands whose sum
// is that operand exactly: x = hi + lo with hi = E4M3(x) and lo = E4M3(x - hi).  A bf16
// value has 8 significant bits and hi takes the top 4 (rounded), so x - hi is an integer
// multiple of x's last bit of at most 4 bits, which E4M3 holds exactly while it stays
// above the E4M3 subnormal step 2^-9.  Each row of the query is first scaled by a power
// of two 2^sh that puts its largest magnitude in [128, 256) (the factor 2^-sh goes into
// the row's score scale), so every element of magnitude at least 2^-2 after scaling, i.e.
// 2^-9 of the row's largest, is split exactly; smaller ones keep an absolute error of at
// most 2^-10 after scaling, under 2^-17 of the row's largest.
// The FP8 path works on 64-token tiles (two halves of 32, M-blocks of the score product):
//   scores  S^T = K . (Q_hi + Q_lo)^T: per half, 9 K-steps of 64 dims, each raw K operand
//           read from LDS once and used by two MFMA 32x32x64 (hi, then lo)
//   output  O^T += V^T . (P'_hi + P'_lo)^T 2^-e: per 32 dims, two scaled MFMA 32x32x64 on
//           one V^T operand that holds each of the tile's 64 tokens once (see
//           split_vt_offsets for the operand layout), B = P'_hi, then B = P'_lo.  V^T is
//           read from the raw tile with the 8-bit LDS transpose read, so no tile is ever
//           converted to bf16.
// The softmax weights are split the same way after a per-row, per-tile power-of-two
// scale 2^e that puts the tile's largest weight in [2^7, 2^8) (split_piece64): P' = hi +
// lo to about 8 significant bits, like bf16, within E4M3's range, and the output MFMA's
// E8M0 operand scale takes 2^e out again.
// ------------------------------------------------------------------------------------

// two floats -> two E4M3 codes (nearest, ties to even) in half-word `hw` of w
// Written as inline assembly: the compiler's handling of these converts' half-word
// select (the other half kept from the destination) merges unrelated conversions.
template <bool HW>
__device__ __forceinline__ unsigned e4m3_pair(unsigned w, float a, float b) {
  if (HW) asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(w) : "v"(a), "v"(b));
  else asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, 1.0" : "=v"(w) : "v"(a), "v"(b));
  return w;
}
template <bool HW>
__device__ __forceinline__ f32x2 e4m3_pair_value(unsigned w) {
  f32x2 r;
  if (HW) asm("v_cvt_scalef32_pk_f32_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  else asm("v_cvt_scalef32_pk_f32_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}
// both: E4M3 codes of (a, b) into half-word HW of *hc, of the remainders into *lc
template <bool HW>
__device__ __forceinline__ void e4m3_split_pair(unsigned& hc, unsigned& lc, float a, float b) {
  hc = e4m3_pair<HW>(hc, a, b);
  const f32x2 hv = e4m3_pair_value<HW>(hc);
  lc = e4m3_pair<HW>(lc, a - hv[0], b - hv[1]);
}

// Query row of this lane as the split operands of the score product: K-step k covers dims
// 64k .. 64k+63, lane half h dims 64k + 32h .. + 31 as bytes 0..31 (as in qk_tile_f8).
// Returns sh (the row's values were multiplied by 2^sh).  The lane's 288 values are loaded
// at once; their largest magnitude (of lanes l and l ^ 32) sets sh, then each K-step is
// converted (its raw registers are free again once its codes exist).
__device__ __forceinline__ int q_split(const uint16_t* qrow, const uint16_t* prow, int lh, i32x8* qh, i32x8* ql) {
  u32x4 raw[36];
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int d = 64 * k + 32 * lh;
    const u32x4* src = reinterpret_cast<const u32x4*>((d < kLatent) ? qrow + d : prow + (d - kLatent));
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) raw[4 * k + w4] = src[w4];
  }
  unsigned amax = 0;  // largest |bf16| bit pattern (ordered like the magnitudes)
#pragma unroll
  for (int j = 0; j < 36; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = max(amax, max(raw[j][e] & 0x7FFFu, (raw[j][e] >> 16) & 0x7FFFu));
  {
    auto r = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
    amax = max(r[0], r[1]);
  }
  // 2^sh * amax in [128, 256) (bounded so that 2^sh and 2^-sh stay normal floats)
  const int sh = amax ? min(max(7 - ((int)(amax >> 7) - 127), -126), 126) : 0;
  const float sc = __uint_as_float((unsigned)(sh + 127) << 23);
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    i32x8 h = {}, l = {};
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const u32x4 r4 = raw[4 * k + w4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // dims 8 w4 + 2e, 8 w4 + 2e + 1 -> bytes of dword 2 w4 + e / 2
        const float a = __uint_as_float(r4[e] << 16) * sc, b = __uint_as_float(r4[e] & 0xFFFF0000u) * sc;
        const int dw = 2 * w4 + (e >> 1);
        unsigned hc = (unsigned)h[dw], lc = (unsigned)l[dw];
        if (e & 1) e4m3_split_pair<true>(hc, lc, a, b);
        else e4m3_split_pair<false>(hc, lc, a, b);
        h[dw] = (int)hc;
        l[dw] = (int)lc;
      }
    }
    qh[k] = h;
    ql[k] = l;
  }
  return sh;
}

// FP8 query (cache format 3): the query row rounded to E4M3 once per segment, in the
// operand layout of qk_tile_f8 (K-step k: dims 64k + 32h .. + 31 as bytes 0..31): each
// value saturated at +-448 (a NaN to 448 with its sign), then the hardware conversion
// (nearest, ties to even).  For every bf16 input this gives the codes of the cache
// append's encoder (e4m3_code): a probe compared all 65536 patterns.
__device__ __forceinline__ void q_round_e4m3(const uint16_t* qrow, const uint16_t* prow, int lh, i32x8* q8) {
  auto sat = [](float x) { return copysignf(fminf(fabsf(x), 448.0f), x); };
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int d = 64 * k + 32 * lh;
    const u32x4* src = reinterpret_cast<const u32x4*>((d < kLatent) ? qrow + d : prow + (d - kLatent));
    i32x8 v;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const u32x4 raw = src[w4];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {  // dims 8 w4 + 2e .. + 3 -> dword 2 w4 + e / 2
        unsigned c = e4m3_pair<false>(0u, sat(__uint_as_float(raw[e] << 16)),
                                      sat(__uint_as_float(raw[e] & 0xFFFF0000u)));
        c = e4m3_pair<true>(c, sat(__uint_as_float(raw[e + 1] << 16)),
                            sat(__uint_as_float(raw[e + 1] & 0xFFFF0000u)));
        v[2 * w4 + e / 2] = (int)c;
      }
    }
    q8[k] = v;
  }
}

// ------------------------------------------------------------------------------------
// FP8 tiles of 64 tokens.  A raw tile is two 32-token halves, each in the load_fp8_raw
// layout (half h at byte 18432 h); M-block m of the score product is half m.  One
// 64-token tile per iteration halves the per-token cost of everything that happens once
// per tile (loop, block-table reads, waits, barrier, the softmax's row reductions), and
// each V^T operand feeds two output MFMAs (P'_hi, then P'_lo) instead of carrying its
// tokens twice.
// ------------------------------------------------------------------------------------

constexpr int kT8 = 64;                        // tokens per FP8 tile
constexpr int kHalfBytes = kFp8RawBytes;       // 18432: one 32-token half
constexpr int kT8Bytes = 2 * kHalfBytes;       // 36864
constexpr int kT8Ahead = 2;                    // loads of tile i + 2 go out in iteration i
constexpr int kT8Loads = kFp8Loads / 2;        // 9 load instructions per wavefront and tile

// Raw 64-token tile starting at token tb.  Half h's 18 load instructions are dealt to the
// wavefronts as in load_fp8_raw but rotated by 2h, so every wavefront issues nine.  A
// second half that starts past the request's last token reloads the first half (its
// scores are masked), so every address stays inside the request's pages.  e0, e1: the
// block-table entries of the halves' first tokens (e1 = e0 if the second half reloads).
__device__ __forceinline__ int half1_start(const Src& S, int tb) { return tb + 32 < S.n ? tb + 32 : tb; }
__device__ __forceinline__ void load_fp8_tile64(const Src& S, int tb, int e0, int e1, uint32_t st, int wave,
                                                int lane) {
  load_fp8_raw(S, tb, page_start(S, e0), st, wave, lane);
  load_fp8_raw(S, half1_start(S, tb), page_start(S, e1), st + kHalfBytes, (wave + 2) & 3, lane);
}

// Scores of one 64-token tile on the split query: S^T_m = K_m . Q_hi^T + K_m . Q_lo^T for
// the halves m = 0, 1 (accumulated in s0, s1).  Per K-step of 64 dims: the raw K operand
// of each half (chunks 2h, 2h+1 of token row l % 32 at f[e] + 2048 k + 18432 m), read from
// LDS once and used by the hi and the lo MFMA.  Operand buffers are two fixed sets of
// 2 x 8 registers (v224..v255); the reads of a half run one M-block ahead, a buffer is
// refilled only after two later MFMAs were issued, and every wait counts the reads issued
// after the ones it needs (LDS reads complete in order).  The closing s_nop run covers the
// wait states before vector instructions may read s0 and s1.
__device__ __forceinline__ void qk_tile64_split(const i32x8* qh, const i32x8* ql, uint32_t raw, const uint32_t* f,
                                                f32x16& s0, f32x16& s1) {
  const uint32_t f0 = raw + f[0], f1 = raw + f[1];
  asm volatile(
      "ds_read_b128 v[224:227], %[f0] offset:0\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:0\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:18432\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:18432\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:2048\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:2048\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[h0], 0\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[l0], %[s0]\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:20480\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:20480\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[h0], 0\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[l0], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:4096\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:4096\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[h1], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[l1], %[s0]\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:22528\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:22528\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[h1], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[l1], %[s1]\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:6144\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:6144\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[h2], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[l2], %[s0]\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:24576\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:24576\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[h2], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[l2], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:8192\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:8192\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[h3], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[l3], %[s0]\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:26624\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:26624\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[h3], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[l3], %[s1]\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:10240\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:10240\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[h4], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[l4], %[s0]\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:28672\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:28672\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[h4], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[l4], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:12288\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:12288\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[h5], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[l5], %[s0]\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:30720\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:30720\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[h5], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[l5], %[s1]\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:14336\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:14336\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[h6], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[l6], %[s0]\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:32768\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:32768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[h6], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[l6], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:16384\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:16384\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[h7], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[l7], %[s0]\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:34816\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:34816\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[h7], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[l7], %[s1]\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[h8], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[l8], %[s0]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[h8], %[s1]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[l8], %[s1]\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : [s0] "=&v"(s0), [s1] "=&v"(s1)
      : [f0] "v"(f0), [f1] "v"(f1),
        [h0] "v"(qh[0]), [h1] "v"(qh[1]), [h2] "v"(qh[2]), [h3] "v"(qh[3]), [h4] "v"(qh[4]),
        [h5] "v"(qh[5]), [h6] "v"(qh[6]), [h7] "v"(qh[7]), [h8] "v"(qh[8]),
        [l0] "v"(ql[0]), [l1] "v"(ql[1]), [l2] "v"(ql[2]), [l3] "v"(ql[3]), [l4] "v"(ql[4]),
        [l5] "v"(ql[5]), [l6] "v"(ql[6]), [l7] "v"(ql[7]), [l8] "v"(ql[8])
      : "memory", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235",
        "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248",
        "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}

// Scores of one 64-token tile with the FP8 query (cache format 3): one MFMA per half and
// K-step, A = the raw K codes, B = the query codes.  The matrix core pairs equal byte
// positions of equal lane halves, so query and key take the same dims per byte.  Three
// fixed buffer sets of 2 x 8 registers (v208..v255), reads two K-steps ahead, a set
// refilled two MFMAs after its last use.
__device__ __forceinline__ void qk_tile64_f8(const i32x8* q, uint32_t raw, const uint32_t* f, f32x16& s0,
                                             f32x16& s1) {
  const uint32_t f0 = raw + f[0], f1 = raw + f[1];
  asm volatile(
      "ds_read_b128 v[208:211], %[f0] offset:0\n\t"
      "ds_read_b128 v[212:215], %[f1] offset:0\n\t"
      "ds_read_b128 v[216:219], %[f0] offset:18432\n\t"
      "ds_read_b128 v[220:223], %[f1] offset:18432\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:2048\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:2048\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:20480\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:20480\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[208:215], %[q0], 0\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[216:223], %[q0], 0\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:4096\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:4096\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:22528\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:22528\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[q1], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[q1], %[s1]\n\t"
      "ds_read_b128 v[208:211], %[f0] offset:6144\n\t"
      "ds_read_b128 v[212:215], %[f1] offset:6144\n\t"
      "ds_read_b128 v[216:219], %[f0] offset:24576\n\t"
      "ds_read_b128 v[220:223], %[f1] offset:24576\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[q2], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[q2], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:8192\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:8192\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:26624\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:26624\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[208:215], %[q3], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[216:223], %[q3], %[s1]\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:10240\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:10240\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:28672\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:28672\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[q4], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[q4], %[s1]\n\t"
      "ds_read_b128 v[208:211], %[f0] offset:12288\n\t"
      "ds_read_b128 v[212:215], %[f1] offset:12288\n\t"
      "ds_read_b128 v[216:219], %[f0] offset:30720\n\t"
      "ds_read_b128 v[220:223], %[f1] offset:30720\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[q5], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[q5], %[s1]\n\t"
      "ds_read_b128 v[224:227], %[f0] offset:14336\n\t"
      "ds_read_b128 v[228:231], %[f1] offset:14336\n\t"
      "ds_read_b128 v[232:235], %[f0] offset:32768\n\t"
      "ds_read_b128 v[236:239], %[f1] offset:32768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[208:215], %[q6], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[216:223], %[q6], %[s1]\n\t"
      "ds_read_b128 v[240:243], %[f0] offset:16384\n\t"
      "ds_read_b128 v[244:247], %[f1] offset:16384\n\t"
      "ds_read_b128 v[248:251], %[f0] offset:34816\n\t"
      "ds_read_b128 v[252:255], %[f1] offset:34816\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[224:231], %[q7], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[232:239], %[q7], %[s1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s0], v[240:247], %[q8], %[s0]\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %[s1], v[248:255], %[q8], %[s1]\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : [s0] "=&v"(s0), [s1] "=&v"(s1)
      : [f0] "v"(f0), [f1] "v"(f1),
        [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]),
        [q5] "v"(q[5]), [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8])
      : "memory", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219",
        "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232",
        "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245",
        "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255");
}

// Operand layout of MFMA 32x32x64 with 8-bit operands (probed on the box with one-hot
// operands and distinct E8M0 scales): byte t of lane half h is element
// k = 32 (t / 16) + 16 h + t % 16, so bytes 0..15 of both halves form the first 32-element
// scale block and bytes 16..31 the second; the scale of block b for row (A) or column
// (B) j comes from lane 32 b + j.
//
// Output product of a 64-token tile, per 32 dims: two MFMAs on the same V^T operand, one
// with B = P'_hi, one with B = P'_lo.  Lane half h's bytes 0..15 are the 16 tokens of half
// 0 whose scores that lane half holds (tokens 4h + 8g + r, g, r = 0..3, in the scores'
// register order) and bytes 16..31 the same positions in half 1, so P needs no lane
// exchange and V^T carries every token once.  V^T of dim block db (dims 32 db + l % 32)
// takes four 8-bit transpose reads per lane: read (t, m) covers tokens 4h + 16t +
// {0..3, 8..11} of half m; in each 16-lane group g, lane s addresses token
// 4h + 16t + u % 4 + 8 (u / 4), u = s / 2, and dims 32 db + 16 (g % 2) + 8 (s % 2) .. + 8
// (raw chunk 2 db + g % 2, whose position in the row is swizzled with sswz), and lane j
// receives dim 32 db + 16 (g % 2) + j of the 8 tokens.  vs[2t + (db & 1)] is the lane's
// offset inside chunk group db / 2 (odd blocks flip position bit 1, byte-offset bit 5).
__device__ __forceinline__ void split_vt_offsets(int lane, int* vs) {
  const int g = lane >> 4, s = lane & 15, h = lane >> 5, u = s >> 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = 4 * h + 16 * t + (u & 3) + 8 * (u >> 2);
    const int off = 64 * tok + 16 * ((g & 1) ^ sswz(tok)) + 8 * (s & 1);
    vs[2 * t] = off;
    vs[2 * t + 1] = off ^ 32;
  }
}
__device__ __forceinline__ i32x8 vt64_read(const uint32_t* base, int db) {
  i32x2 r[4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      r[2 * m + t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          at<i32x2>(base[2 * t + (db & 1)] + 2048 * (db >> 1) + kHalfBytes * m));
  return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

// The lane id, computed where it is called (a volatile statement is never moved out of a
// loop), for per-lane offsets that are cheaper to recompute than to keep in registers.
__device__ __forceinline__ int lane_id_here() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

// Output MFMA of the FP8 path, c += V^T . P'^T: A = V^T codes at unit scale (E8M0 127 in
// ua), B = P' codes with this row's E8M0 scale sb.  Written as an assembly statement,
// which stays where the schedule puts it (the compiler sinks the builtin form past the
// softmax work it is meant to interleave with).  Hazards the compiler cannot see: a
// vector instruction writing an operand needs two wait states before the MFMA reads it
// (NOP: the first MFMA of a phase, whose P operand may just have been assembled), and a
// read of the accumulators after the last MFMA waits for it (mfma_drain).
template <bool NOP = false>
__device__ __forceinline__ void mfma_f8s(f32x16& c, const i32x8& a, const i32x8& b, int ua, int sb) {
  if (NOP)
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(c) : "v"(a), "v"(b), "v"(ua), "v"(sb));
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(c) : "v"(a), "v"(b), "v"(ua), "v"(sb));
}
// wait states (more than the 16-pass MFMA's 19) before an accumulator may be read
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Online softmax of one 64-token tile, in 32 pieces (one per output MFMA).  x: raw scores
// of this lane (x[16 m + v]: half m, token 8 (v / 4) + 4 (l / 32) + v % 4 of it, row
// l % 32), masked ones -inf; c > 0 the row's score scale in log2 units.  Weights are
// p = 2^(x c - m) with the reference m moved only when the tile's max exceeds it by more
// than 8, and then to that max - 1, so p <= 2^8 and the row's max may grow by 7 before the
// accumulators need rescaling (any row of the wavefront then rescales all 256
// accumulators).  Each row's weights of the tile are carried as p' = p 2^e, with the
// integer e chosen so that the tile's largest p' lies in [2^7, 2^8): p' = hi + lo, hi and
// lo E4M3, so every weight within 2^-8 of the tile's largest keeps 8 significant bits and
// smaller ones an absolute error of at most 2^-10, i.e. 2^-17 of the tile's largest,
// however far the tile lies below the row's reference.  The output MFMAs undo 2^e with the
// B operand's E8M0 scale.  Output: alpha (factor for the accumulators before this tile's
// product), the codes of hi (ph) and lo (pl), dword j holding values 4j .. 4j+3 (so
// bytes 0..15 are half 0's values, bytes 16..31 half 1's), and sb, the E8M0 code of 2^-e.
struct SplitPieces {
  float mt, m_new, ex, nm, acc, esc;
  bool need;
};
__device__ __forceinline__ void split_piece64(int k, Softmax& S, float* x, float c, SplitPieces& w, unsigned* ph,
                                              unsigned* pl, float& alpha, int& sb) {
  auto split4 = [&](int j) {  // values 4j .. 4j+3 -> dword j of the hi and lo codes
    unsigned hc = 0, lc = 0;
    e4m3_split_pair<false>(hc, lc, x[4 * j], x[4 * j + 1]);
    e4m3_split_pair<true>(hc, lc, x[4 * j + 2], x[4 * j + 3]);
    ph[j] = hc;
    pl[j] = lc;
  };
  if (k == 0) {
    w.mt = max3(max3(max3(max3(x[0], x[1], x[2]), x[3], x[4]), x[5], x[6]), x[7], x[8]);
  } else if (k == 1) {
    w.mt = max3(max3(max3(max3(max3(w.mt, x[9], x[10]), x[11], x[12]), x[13], x[14]), x[15], x[16]), x[17], x[18]);
  } else if (k == 2) {
    w.mt = max3(max3(max3(max3(max3(max3(w.mt, x[19], x[20]), x[21], x[22]), x[23], x[24]), x[25], x[26]), x[27],
                     x[28]),
                x[29], max3(x[30], x[31], x[31]));
  } else if (k == 3) {
    w.mt = pair_max(w.mt) * c;  // -inf stays -inf (c > 0)
  } else if (k == 4) {
    w.need = w.mt > S.m_used + 8.0f;
    w.m_new = w.need ? w.mt - 1.0f : S.m_used;
    w.ex = __builtin_amdgcn_exp2f(S.m_used - w.m_new);
  } else if (k == 5) {
    // (while no token has been seen the accumulators are zero and need no factor)
    alpha = (w.need && S.m_used != -INFINITY) ? w.ex : 1.0f;
    S.l_sum *= alpha;
    S.m_used = w.m_new;
    // e = 7 - floor(tile max - reference), within [-1, 100]; a row with no visible token
    // in this tile (mt = -inf, NaN difference) takes the bound, its weights are all 0
    const float d = fmaxf(w.mt - w.m_new, -100.0f);
    const int e = min(7 - (int)floorf(d), 100);
    w.esc = __uint_as_float((unsigned)(127 - e) << 23);  // 2^-e
    w.nm = (w.m_new == -INFINITY) ? 0.f : (float)e - w.m_new;
    sb = 127 - e;
    w.acc = 0.f;
  } else if (k >= 6 && k < 22) {
    const int v = 2 * (k - 6);
    x[v] = __builtin_amdgcn_exp2f(fmaf(x[v], c, w.nm));
    x[v + 1] = __builtin_amdgcn_exp2f(fmaf(x[v + 1], c, w.nm));
    w.acc += x[v];
    w.acc += x[v + 1];
    if (k >= 8 && (k & 1) == 0) split4((k - 8) / 2);  // values 4j .. 4j+3 are done from step 7 + 2j on
  } else if (k == 22) {
    split4(7);
    S.l_sum = fmaf(w.acc, w.esc, S.l_sum);  // sum of p = 2^-e sum of p'
  }
}

// Output product of tile i-1 (raw tile `raw`, P' codes ph/pl with scale sbp) for the FP8
// path, with the softmax of tile i in pieces between its 32 MFMAs; V^T reads run kAhead
// dim blocks ahead.
template <int kAhead>
__device__ __forceinline__ void output_phase64(f32x16* o, uint32_t raw, const unsigned* ph, const unsigned* pl,
                                               int sbp, const int* vs, float* x, Softmax& S, float c, unsigned* nh,
                                               unsigned* nl, float& alpha, int& sb) {
  uint32_t base[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) base[v] = raw + vs[v];
  const i32x8 bh = {(int)ph[0], (int)ph[1], (int)ph[2], (int)ph[3], (int)ph[4], (int)ph[5], (int)ph[6], (int)ph[7]};
  const i32x8 bl = {(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3], (int)pl[4], (int)pl[5], (int)pl[6], (int)pl[7]};
  const int ua = 127;
  SplitPieces w;
  i32x8 va[kDimBlocks];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) va[k] = vt64_read(base, k);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db) {
    if (db == 0) mfma_f8s<true>(o[db], va[db], bh, ua, sbp);
    else mfma_f8s(o[db], va[db], bh, ua, sbp);
    split_piece64(2 * db, S, x, c, w, nh, nl, alpha, sb);
    __builtin_amdgcn_sched_barrier(0);
    mfma_f8s(o[db], va[db], bl, ua, sbp);
    if (db + kAhead < kDimBlocks) va[db + kAhead] = vt64_read(base, db + kAhead);
    split_piece64(2 * db + 1, S, x, c, w, nh, nl, alpha, sb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The softmax of one tile on its own (the first tile of a range).
__device__ __forceinline__ float softmax64(Softmax& S, float* x, float c, unsigned* nh, unsigned* nl, int& sb) {
  SplitPieces w;
  float alpha = 1.f;
#pragma unroll
  for (int k = 0; k < 2 * kDimBlocks; ++k) split_piece64(k, S, x, c, w, nh, nl, alpha, sb);
  return alpha;
}

// The output product of one tile on its own (the last tile of a range); the accumulators
// may be read right after it.
__device__ __forceinline__ void pv64(f32x16* o, uint32_t raw, const unsigned* ph, const unsigned* pl, int sbp,
                                     const int* vs) {
  uint32_t base[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) base[v] = raw + vs[v];
  const i32x8 bh = {(int)ph[0], (int)ph[1], (int)ph[2], (int)ph[3], (int)ph[4], (int)ph[5], (int)ph[6], (int)ph[7]};
  const i32x8 bl = {(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3], (int)pl[4], (int)pl[5], (int)pl[6], (int)pl[7]};
  const int ua = 127;
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db) {
    const i32x8 va = vt64_read(base, db);
    if (db == 0) mfma_f8s<true>(o[db], va, bh, ua, sbp);
    else mfma_f8s(o[db], va, bh, ua, sbp);
    mfma_f8s(o[db], va, bl, ua, sbp);
  }
  mfma_drain();
}

// ------------------------------------------------------------------------------------
// One token range of one request: Q load, pipelined tile loop, partial epilogue.
// D: wavefronts per block of 32 rows.  With D = 1 a workgroup holds 128 rows, one block
// per wavefront; with few rows (D = 2: at most 64, D = 4: at most 32) the D wavefronts of
// a row block share it by output dims, each holding the accumulators of 512 / D of them
// (the scores and the softmax are the same in all D, so they run in each).
// ------------------------------------------------------------------------------------

// The query row (the 36 Q^T operands of this lane, bf16) as f16 operands for the NVFP4
// path: every value times 2^sh, with sh chosen so that the row's largest magnitude (over
// lanes l and l ^ 32, which hold the row's two halves) lands in [2^14, 2^15).  The f16
// values are then exact for every element of at least 2^-17 after scaling, i.e. 2^-31
// of the row's largest (f16 keeps 11 bits down to 2^-14 and 8 bits down to 2^-17).
// Returns the row's score scale in log2 units with 2^-sh taken out (kept positive:
// sm_scale = 0 gives the plain mean).
__device__ __forceinline__ float q_to_f16(bf16x8* q, float score_scale) {
  unsigned amax = 0;  // largest |bf16| bit pattern (ordered like the magnitudes)
#pragma unroll
  for (int k = 0; k < kKSteps; ++k) {
    const u32x4 w = __builtin_bit_cast(u32x4, q[k]);
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = max(amax, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
    amax = max(r[0], r[1]);
  }
  const int sh = amax ? min(max(14 - ((int)(amax >> 7) - 127), -126), 126) : 0;
  const float sc = __uint_as_float((unsigned)(sh + 127) << 23);
#pragma unroll
  for (int k = 0; k < kKSteps; ++k) {
    const u32x4 w = __builtin_bit_cast(u32x4, q[k]);
    u32x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 v = {(_Float16)(__uint_as_float(w[e] << 16) * sc),
                       (_Float16)(__uint_as_float(w[e] & 0xFFFF0000u) * sc)};
      h[e] = __builtin_bit_cast(unsigned, v);
    }
    q[k] = __builtin_bit_cast(bf16x8, h);
  }
  return fmaxf(score_scale * __uint_as_float((unsigned)(127 - sh) << 23), 1e-37f);
}

template <int FMT, bool PAGED, int D = 1>
__device__ __forceinline__ void run_range(const DecodeParams& p, uint32_t smem, int b, int n, int rg, int lt0,
                                          int lt1, int64_t slot) {
  using PP = Pipe<FMT>;
  static_assert(D == 1 || D == 2 || D == 4, "wavefronts per row block");
  static_assert(D == 1 || FMT == kFmtBf16, "shared row blocks on the bf16 cache only");
  constexpr int NB = kDimBlocks / D;                      // dim blocks of this wavefront
  constexpr int kGroupRows = kRowsPerGroup / D;           // rows of a workgroup
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform, and known so
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int rblk = wave % (kWaves / D), dpart = wave / (kWaves / D);
  const int db0 = NB * dpart;                             // first dim block of this wavefront
  const int row0 = rg * kGroupRows;                       // first row of this workgroup
  const int rows_here = min(kGroupRows, p.rows - row0);
  const int my_row = kWaveRows * rblk + lr;               // this lane's row (in the group)
  const int rc = min(row0 + my_row, p.rows - 1);          // rows past the end repeat the last row
  float c = p.score_scale > 0.f ? p.score_scale : 1e-30f;  // sm_scale = 0 gives the plain mean
  const int nt = lt1 - lt0;
  // the NVFP4 cache runs on f16 operands (its dequantised values are exact in f16 and
  // the weights keep 11 bits); the bf16 cache on bf16 operands
  constexpr bool H = FMT == kFmtNvfp4;

  // Q^T operand, row rc: dims 16k + 8 (l / 32) .. + 8
  bf16x8 q[kKSteps];
  {
    const uint16_t* qrow = p.q + ((int64_t)b * p.rows + rc) * kLatent;
    const uint16_t* prow = p.qpe + ((int64_t)b * p.rows + rc) * kRope;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const int d = 16 * k + 8 * lh;
      const uint16_t* src = (d < kLatent) ? qrow + d : prow + (d - kLatent);
      q[k] = *reinterpret_cast<const bf16x8*>(src);
    }
  }
  if constexpr (H) c = q_to_f16(q, p.score_scale);
  // query i of a request sees tokens lo .. vis - 1: vis = n - q_len + i + 1, and lo = 0, or
  // vis - window with a sliding window
  const int vis = max(n - p.q_len + rc / p.H + 1, 0);
  const int lo = p.window > 0 ? max(vis - p.window, 0) : 0;
  int min_vis = vis;  // fewest tokens any row of this wavefront sees: tiles below it need no mask
  int max_lo = lo;    // and the latest first token: tiles from it on need no mask
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    min_vis = min(min_vis, __shfl_xor(min_vis, o));
    max_lo = max(max_lo, __shfl_xor(max_lo, o));
  }

  int ab[4];  // score operand offsets, a_base ^ 32x (see qk_tile)
  {
    const int a_base = 128 * lr + ((lh ^ swz(lr)) << 4);
#pragma unroll
    for (int x = 0; x < 4; ++x) ab[x] = a_base ^ (32 * x);
  }
  // transpose reads: in a group of 16 lanes (g = l / 16, j = l % 16), lane j addresses
  // token 8 (g >> 1) + 4e + j / 4 and dims 16 (g & 1) + 4 (j % 4) .. + 4; lane i of the
  // group then receives dim 16 (g & 1) + i of those four tokens
  int vb[4];  // transpose-read offsets [e][db & 1] (see pv_tile)
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tok = 8 * (g >> 1) + 4 * e + (j >> 2);
      const int dim = 16 * (g & 1) + 4 * (j & 3);
      const int v_off = tile_off(tok, dim >> 3) + 2 * (dim & 7);
      vb[2 * e] = v_off;
      vb[2 * e + 1] = v_off ^ 64;
    }
  }

  f32x16 o[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) o[db] = f32x16{};
  Softmax S{-INFINITY, 0.f, 0.f};
  unsigned pp[8];

  const Src src{&p, b, n};
  const int nloads = (PP::kLoads - wave + kWaves - 1) / kWaves;  // load instructions per tile here
  // buffer addresses go through readfirstlane, which keeps the loop optimiser from
  // turning every per-lane LDS address into an induction variable of its own
  auto tile_buf = [&](int i) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem + (uint32_t)((i % PP::kTiles) * PP::kStride)));
  };
  auto raw_buf = [&](int i) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(smem + (uint32_t)(PP::kTiles * PP::kStride + (i % (PP::kRaw ? PP::kRaw : 1)) * PP::kRawBytes)));
  };
  auto entry = [&](int i) {  // block-table entry of tile i (paged caches)
    return PAGED ? table_entry(src, (lt0 + min(i, nt - 1)) * kTileTokens) : 0;
  };
  auto issue = [&](int i, int e) {  // loads of tile i, whose block-table entry is e
    const int tb = (lt0 + i) * kTileTokens;
    const uint8_t* pg = PAGED ? page_start(src, e) : nullptr;
    if (FMT == kFmtBf16) load_bf16_tile<PAGED>(src, tb, pg, tile_buf(i), wave, lane);
    else load_nvfp4_raw(src, tb, pg, raw_buf(i), wave, lane);
  };
  int e_next = 0;  // block-table entry of tile i + kAhead, read one tile early
  auto dequant = [&](int i) {  // raw tile i -> its f16 buffer
    if (FMT == kFmtNvfp4) dequant_nvfp4(raw_buf(i), tile_buf(i), tid);
  };

  // Scores of the latest tile (masked); their softmax runs in the next tile's score block,
  // so they stay in registers until then.
  float x[16];

  // one tile; FIRST: there is no previous tile to multiply
  // loads run kAhead tiles ahead; a bf16 range of at most kTiles tiles loads them all at
  // once (no buffer is reused, so their latencies overlap)
  const int ahead = (FMT == kFmtBf16 && nt <= PP::kTiles) ? nt : PP::kAhead;
  auto body = [&](int i, auto FIRST) {
    constexpr bool first = decltype(FIRST)::value;
    const bool more = i + ahead < nt;
    if (more) {
      issue(i + ahead, e_next);
      e_next = entry(i + ahead + 1);
    }
    f32x16 s;
    if (first) {
      s = qk_tile<H>(q, tile_buf(i), ab);
    } else {
      // scores of tile i, softmax of tile i-1 (x) -> P^T in pp and its factor
      float alpha;
      s = qk_softmax_tile<H>(q, tile_buf(i), ab, x, S, c, pp, alpha);
      if (__any(alpha != 1.f)) rescale<NB>(o, alpha);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = s[v];
    const int tbase = (lt0 + i) * kTileTokens;
    if (tbase + kTileTokens > min_vis || tbase < max_lo) {
      // value v (token tbase + 4 (l / 32) + 8 (v/4) + v%4 of the lane) visible iff in [flo, lim)
      const int lim = vis - tbase - 4 * lh, flo = lo - tbase - 4 * lh;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 8 * (v >> 2) + (v & 3);
        x[v] = (t < lim && t >= flo) ? x[v] : -INFINITY;
      }
    }
    // past the last tile the dequantisation only rewrites an unused buffer; after the
    // first tile it runs spread over the output phase
    if (first) {
      if (FMT == kFmtNvfp4) dequant(i + 1);
    } else if constexpr (FMT == kFmtNvfp4) {
      NvDequant nv(raw_buf(i + 1), tile_buf(i + 1), tid);
      output_phase<kDimBlocks, true>(o, tile_buf(i - 1), pp, vb, &nv);
    } else {
      output_phase<NB>(o, tile_buf(i - 1), pp, vb, nullptr, db0);
    }
    // the loads the next tile depends on: bf16 tile i+1, raw NVFP4 tile i+2; the tiles
    // issued after it may stay in flight
    const int need = FMT == kFmtBf16 ? i + 1 : i + 2;
    wait_vmcnt(max(min(nt - 1, i + ahead) - need, 0) * nloads);
    __syncthreads();
  };

  if (nt > 0) {
    const int pro = min(nt, ahead);
    for (int k = 0; k < pro; ++k) issue(k, entry(k));
    e_next = entry(ahead);
    wait_vmcnt((pro - 1) * nloads);  // tile 0
    __syncthreads();
    if (FMT != kFmtBf16) {
      dequant(0);
      wait_vmcnt(max(pro - 2, 0) * nloads);  // raw tile 1
      __syncthreads();
    }
    body(0, std::true_type{});
    for (int i = 1; i < nt; ++i) body(i, std::false_type{});
    const float alpha = softmax_tile<H>(S, x, c, pp);  // the last tile's softmax
    if (__any(alpha != 1.f)) rescale<NB>(o, alpha);
    pv_tile<NB, H>(o, tile_buf(nt - 1), pp, vb, db0);
  }

  // ---- epilogue: normalised partial O and its lse ----
  const float l_tot = pair_sum(S.l_sum);
  const float l_rnd = pair_sum(S.l_rnd);
  const bool ok = l_tot > 0.f;
  if (my_row < rows_here) {
    const int row = row0 + my_row;
    if (lh == 0 && dpart == 0)
      p.lse_part[slot * p.l_slot + (int64_t)row * p.l_row] = ok ? (S.m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
    const float f = ok ? p.v_scale / l_rnd : 0.f;  // normalisation, applied on the way out
    float* orow = p.o_part + slot * p.o_slot + (int64_t)row * p.o_row + 4 * lh + 32 * db0;
    // four dim blocks at a time: 64 values scaled into vector registers, then 16 stores
    // issued back to back
#pragma unroll
    for (int g = 0; g < NB; g += 4) {
      f32x4 t[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int db = g + j / 4, q4 = j % 4;
        t[j] = f32x4{scaled(o[db][4 * q4], f), scaled(o[db][4 * q4 + 1], f), scaled(o[db][4 * q4 + 2], f),
                     scaled(o[db][4 * q4 + 3], f)};
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) *reinterpret_cast<f32x4*>(orow + 32 * (g + j / 4) + 8 * (j % 4)) = t[j];
    }
  }
  __syncthreads();  // the next range reuses the LDS buffers
}

// One token range of one request on the FP8 path (paged FP8 cache, 64-token tiles
// lt0 .. lt1 - 1 of the request): per tile i, the loads of tile i + 2, the scores of tile
// i, then the output product of tile i-1 with the softmax of tile i between its MFMAs,
// then one barrier.  kQ8 (cache format 3): the query rounded to E4M3 instead of split,
// one score MFMA per half and K-step; everything else is the same.
template <bool kQ8>
__device__ __forceinline__ void run_range_fp8(const DecodeParams& p, uint32_t smem, int b, int n, int rg, int lt0,
                                              int lt1, int64_t slot) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int row0 = rg * kRowsPerGroup;
  const int rows_here = min(kRowsPerGroup, p.rows - row0);
  const int my_row = kWaveRows * wave + lr;
  const int rc = min(row0 + my_row, p.rows - 1);  // rows past the end repeat the last row
  const int nt = lt1 - lt0;
  i32x8 qh[9], ql[kQ8 ? 1 : 9];  // the query row, split (q_split) or rounded (q_round_e4m3, in qh)
  float c = 0.f;                  // its score scale (set with the split)

  const int vis = max(n - p.q_len + rc / p.H + 1, 0);
  const int lo = p.window > 0 ? max(vis - p.window, 0) : 0;
  int min_vis = vis, max_lo = lo;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    min_vis = min(min_vis, __shfl_xor(min_vis, o));
    max_lo = max(max_lo, __shfl_xor(max_lo, o));
  }

  // per-lane LDS offsets of the score and transpose reads; recomputed in each tile from the
  // lane id (a few integer instructions) rather than held in registers across the loop
  // (lane_id_here keeps the compiler from hoisting them out of it again)
  auto score_offsets = [&](uint32_t* fq) {
    const int l = lane_id_here(), r = l & 31, h = l >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) fq[e] = 64 * r + 16 * ((2 * h + e) ^ sswz(r));
  };

  f32x16 o[kDimBlocks];
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db) o[db] = f32x16{};
  Softmax S{-INFINITY, 0.f, 0.f};
  unsigned ph[8], pl[8];  // P' codes of the previous tile (hi, lo)
  int sb_prev = 127;      // and their E8M0 scale
  float alpha_prev = 1.f;

  const Src src{&p, b, n};
  auto raw_buf = [&](int i) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem + (uint32_t)((i & 3) * kT8Bytes)));
  };
  static_assert(Pipe<kFmtFp8>::kRaw == 4 && Pipe<kFmtFp8>::kRawBytes == kT8Bytes, "four 64-token raw tiles");
  // block-table entries of tile i's halves (tiles past the range repeat the last one);
  // both are read, even when one page holds the whole tile, so that neither read waits
  // for the other (they are waited for where the next tile's loads use them)
  auto entry0 = [&](int i) { return table_entry(src, (lt0 + min(i, nt - 1)) * kT8); };
  auto entry1 = [&](int i) { return table_entry(src, half1_start(src, (lt0 + min(i, nt - 1)) * kT8)); };
  auto issue = [&](int i, int e0, int e1) {
    load_fp8_tile64(src, (lt0 + i) * kT8, e0, e1, raw_buf(i), wave, lane);
  };
  int en0 = 0, en1 = 0;  // entries of the next tile to load

  auto body = [&](int i, auto FIRST) {
    constexpr bool first = decltype(FIRST)::value;
    float x[32];
    if (i + kT8Ahead < nt) {
      issue(i + kT8Ahead, en0, en1);
      en0 = entry0(i + kT8Ahead + 1);
      en1 = entry1(i + kT8Ahead + 1);
    }
    if (!first && __any(alpha_prev != 1.f)) rescale(o, alpha_prev);
    f32x16 s0, s1;
    {
      uint32_t fq[2];
      score_offsets(fq);
      if constexpr (kQ8) qk_tile64_f8(qh, raw_buf(i), fq, s0, s1);
      else qk_tile64_split(qh, ql, raw_buf(i), fq, s0, s1);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = s0[v];
      x[16 + v] = s1[v];
    }
    const int tbase = (lt0 + i) * kT8;
    if (tbase + kT8 > min_vis || tbase < max_lo) {
      // value 16 m + v: token tbase + 32 m + 8 (v / 4) + 4 (l / 32) + v % 4 of the lane,
      // visible iff in [lo, vis)
      const int lim = vis - tbase - 4 * lh, flo = lo - tbase - 4 * lh;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int t = 32 * (v >> 4) + 8 * ((v >> 2) & 3) + (v & 3);
        x[v] = (t < lim && t >= flo) ? x[v] : -INFINITY;
      }
    }
    unsigned nh[8], nl[8];
    float alpha = 1.f;
    int sbn = 127;
    if (first) {
      alpha = softmax64(S, x, c, nh, nl, sbn);
    } else {
      int vs[4];
      split_vt_offsets(lane_id_here(), vs);
      output_phase64<2>(o, raw_buf(i - 1), ph, pl, sb_prev, vs, x, S, c, nh, nl, alpha, sbn);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ph[k] = nh[k];
      pl[k] = nl[k];
    }
    sb_prev = sbn;
    alpha_prev = alpha;
    // tile i+1 must have landed (its loads were issued one tile ago); the loads of tile
    // i+2 may stay in flight
    static_assert(kT8Ahead == 2 && kT8Loads == 9, "load counts below");
    if (i + kT8Ahead < nt) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // the first tiles' loads go out before the query is read and split, so that their
  // latency and the query's overlap
  const int pro = min(nt, kT8Ahead);
  if (nt > 0) {
    for (int k = 0; k < pro; ++k) issue(k, entry0(k), entry1(k));
    en0 = entry0(kT8Ahead);
    en1 = entry1(kT8Ahead);
  }
  const uint16_t* qrow = p.q + ((int64_t)b * p.rows + rc) * kLatent;
  const uint16_t* prow = p.qpe + ((int64_t)b * p.rows + rc) * kRope;
  if constexpr (kQ8) {
    q_round_e4m3(qrow, prow, lh, qh);
    c = p.score_scale > 0.f ? p.score_scale : 1e-30f;  // sm_scale = 0 gives the plain mean
  } else {
    const int sh = q_split(qrow, prow, lh, qh, ql);
    // score scale of this row in log2 units, with the query's 2^sh taken out; kept positive
    // (sm_scale = 0 gives the plain mean)
    c = fmaxf(p.score_scale * __uint_as_float((unsigned)(127 - sh) << 23), 1e-37f);
  }

  if (nt > 0) {
    if (pro > 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // tile 0
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    body(0, std::true_type{});
    for (int i = 1; i < nt; ++i) body(i, std::false_type{});
    if (__any(alpha_prev != 1.f)) rescale(o, alpha_prev);
    int vs[4];
    split_vt_offsets(lane, vs);
    pv64(o, raw_buf(nt - 1), ph, pl, sb_prev, vs);
  }

  // ---- epilogue: normalised partial O and its lse (normalised by the unrounded sum) ----
  const float l_tot = pair_sum(S.l_sum);
  const bool ok = l_tot > 0.f;
  if (my_row < rows_here) {
    const int row = row0 + my_row;
    if (lh == 0)
      p.lse_part[slot * p.l_slot + (int64_t)row * p.l_row] = ok ? (S.m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
    const float f = ok ? p.v_scale / l_tot : 0.f;
    float* orow = p.o_part + slot * p.o_slot + (int64_t)row * p.o_row + 4 * lh;
#pragma unroll
    for (int g = 0; g < kDimBlocks; g += 4) {
      f32x4 t[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int db = g + j / 4, q4 = j % 4;
        t[j] = f32x4{scaled(o[db][4 * q4], f), scaled(o[db][4 * q4 + 1], f), scaled(o[db][4 * q4 + 2], f),
                     scaled(o[db][4 * q4 + 3], f)};
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) *reinterpret_cast<f32x4*>(orow + 32 * (g + j / 4) + 8 * (j % 4)) = t[j];
    }
  }
  __syncthreads();  // the next range reuses the LDS buffers
}

// A contiguous split of at most four tiles with at most 32 rows (few heads): the four
// wavefronts take one tile each instead of walking the tiles in turn, each with the
// whole 32-row block and all 512 dims (scores, softmax and output product as in
// run_range), so the split costs one tile of latency instead of four.  The four partial
// results (the row's reference max m_w, its sums of p and of bf16(p), and O_w) are then
// merged through the LDS: with M = max m_w each counts 2^(m_w - M) times, O_j = sum of the
// weighted O_w over the weighted sum of bf16(p), lse_j = (M + log2 of the weighted sum of
// p) ln 2.  The exchange takes one round of all 512 dims for at most 16 rows, else two
// rounds of 256; a row of it is padded by 16 bytes so that the 16-byte accesses of
// neighbouring rows fall in different banks.
__device__ __forceinline__ void run_split_tiles_parallel(const DecodeParams& p, uint32_t smem, int b, int lt0,
                                                         int lt1, int64_t slot) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int rows = p.rows;  // at most 32: one block, shared by the four wavefronts
  const int rc = min(lr, rows - 1);
  const float c = p.score_scale > 0.f ? p.score_scale : 1e-30f;  // sm_scale = 0 gives the plain mean
  const int nt = lt1 - lt0;  // 1 .. 4

  bf16x8 q[kKSteps];
  {
    const uint16_t* qrow = p.q + ((int64_t)b * rows + rc) * kLatent;
    const uint16_t* prow = p.qpe + ((int64_t)b * rows + rc) * kRope;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const int d = 16 * k + 8 * lh;
      const uint16_t* src = (d < kLatent) ? qrow + d : prow + (d - kLatent);
      q[k] = *reinterpret_cast<const bf16x8*>(src);
    }
  }
  int ab[4];
  {
    const int a_base = 128 * lr + ((lh ^ swz(lr)) << 4);
#pragma unroll
    for (int x = 0; x < 4; ++x) ab[x] = a_base ^ (32 * x);
  }
  int vb[4];
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tok = 8 * (g >> 1) + 4 * e + (j >> 2);
      const int dim = 16 * (g & 1) + 4 * (j & 3);
      const int v_off = tile_off(tok, dim >> 3) + 2 * (dim & 7);
      vb[2 * e] = v_off;
      vb[2 * e + 1] = v_off ^ 64;
    }
  }

  // every tile's loads at once (the usual split of load instructions over wavefronts)
  const Src src{&p, b, p.S};
  auto tile_buf = [&](int i) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem + (uint32_t)(i * kTileBytes))); };
  for (int i = 0; i < nt; ++i) load_bf16_tile<false>(src, (lt0 + i) * kTileTokens, nullptr, tile_buf(i), wave, lane);
  wait_vmcnt(0);
  __syncthreads();

  f32x16 o[kDimBlocks];
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db) o[db] = f32x16{};
  Softmax S{-INFINITY, 0.f, 0.f};
  if (wave < nt) {
    const uint32_t tile = tile_buf(wave);
    const f32x16 s = qk_tile(q, tile, ab);
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = s[v];
    const int tbase = (lt0 + wave) * kTileTokens;
    if (tbase + kTileTokens > p.S) {  // the sequence's last tile: tokens from S on are masked
      const int lim = p.S - tbase - 4 * lh;
#pragma unroll
      for (int v = 0; v < 16; ++v) x[v] = (8 * (v >> 2) + (v & 3) < lim) ? x[v] : -INFINITY;
    }
    unsigned pp[8];
    softmax_tile(S, x, c, pp);
    pv_tile<kDimBlocks>(o, tile, pp, vb, 0);
  }
  const float lsum = pair_sum(S.l_sum), lrnd = pair_sum(S.l_rnd);
  __syncthreads();  // every tile has been read: the buffers take the exchange

  const int R = rows <= 16 ? 1 : 2;                 // rounds
  const int DR = kLatent / R;                       // dims per round
  const int RS = DR + 4;                            // exchange row stride (floats)
  const int XR = R == 1 ? 16 : 32;                  // rows kept per wavefront
  LDS_AS float* xl = at<float>(smem);              // [4][XR][RS]
  LDS_AS float* st = at<float>(smem + 136 * 1024);  // [4][32][3]: m, sum p, sum bf16(p)
  if (lh == 0) {
    st[(wave * 32 + lr) * 3 + 0] = S.m_used;
    st[(wave * 32 + lr) * 3 + 1] = lsum;
    st[(wave * 32 + lr) * 3 + 2] = lrnd;
  }
  const int CPW = DR / 16;        // 4-dim chunks per wavefront and row in the merge
  const int RSTEP = 64 / CPW;     // rows a wavefront's lanes cover at once
  const int cc = lane % CPW, r0 = lane / CPW;
  for (int r = 0; r < R; ++r) {
    if (lr < rows && lr < XR) {
#pragma unroll
      for (int db = 0; db < kDimBlocks; ++db) {
        if (db / (kDimBlocks / R) != r) continue;
        const int dl = 32 * (db % (kDimBlocks / R)) + 4 * lh;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<LDS_AS f32x4*>(xl + (wave * XR + lr) * RS + dl + 8 * q4) =
              f32x4{o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]};
      }
    }
    __syncthreads();
    for (int row = r0; row < rows; row += RSTEP) {
      float m[4], a[4];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m[w] = st[(w * 32 + row) * 3];
        M = fmaxf(M, m[w]);
      }
      float l_tot = 0.f, l_rnd = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a[w] = m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[w] - M);
        l_tot += a[w] * st[(w * 32 + row) * 3 + 1];
        l_rnd += a[w] * st[(w * 32 + row) * 3 + 2];
      }
      const bool ok = l_tot > 0.f;
      const float f = ok ? p.v_scale / l_rnd : 0.f;
      const int dloc = (DR / 4) * wave + 4 * cc;  // this lane's 4 dims within the round
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += a[w] * *reinterpret_cast<LDS_AS f32x4*>(xl + (w * XR + row) * RS + dloc);
      *reinterpret_cast<f32x4*>(p.o_part + slot * p.o_slot + (int64_t)row * p.o_row + r * DR + dloc) = acc * f;
      if (r == 0 && wave == 0 && cc == 0)
        p.lse_part[slot * p.l_slot + (int64_t)row * p.l_row] = ok ? (M + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    __syncthreads();  // the next round rewrites the exchange
  }
}

// ------------------------------------------------------------------------------------
// decode kernels
// ------------------------------------------------------------------------------------

// Contiguous: U = row_groups * num_splits * B work items (row group of 128 / D rows,
// split j, request b); split j covers [j*L, min((j+1)*L, S)).  Workgroup ids are dealt
// round-robin over the 8 XCDs, so id -> item is XCD-aware: XCD x takes the consecutive
// items x * per .. x * per + per - 1 of the (request, split, row group) order, and the
// splits of one request share that XCD's L2 (the query is read from HBM once per request
// rather than once per split).  The grid holds 8 * per ids; ids past U exit.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_contig_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<kFmtBf16>()];
  const int R = p.row_groups, U = R * p.num_splits * p.B, per = (U + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= U) return;
  const int rg = u % R, j = (u / R) % p.num_splits, b = u / (R * p.num_splits);
  const int t0 = j * p.kv_len_per_split;
  const int t1 = min(t0 + p.kv_len_per_split, p.S);
  // slot b*H*NS + j with row = head addresses o_part [B, H, NS, 512]
  const int lt0 = t0 / kTileTokens, lt1 = (t1 + kTileTokens - 1) / kTileTokens;
  const int64_t slot = (int64_t)b * p.rows * p.num_splits + j;
  if constexpr (D == 4) {
    if (lt1 - lt0 <= kWaves) {  // few heads and a short split: one tile per wavefront
      run_split_tiles_parallel(p, lds_addr((lds_ptr)smem), b, lt0, lt1, slot);
      return;
    }
  }
  run_range<kFmtBf16, false, D>(p, lds_addr((lds_ptr)smem), b, p.S, rg, lt0, lt1, slot);
}

// Paged: the batch's tiles (request b has ceil(n_b / T), T = 32, or 64 for the FP8
// formats) are cut into num_splits contiguous ranges of about equal cost, one workgroup
// per range and row group (in the XCD-aware order below).  A
// request with tiles costs them plus kSegmentCost: on the cost axis it spans its
// overhead part, then its tiles, and range w takes the tiles that fall in
// [w W / NS, (w + 1) W / NS) of the total cost W.  A range covering parts of several
// requests runs one segment per request; segment (w, b) writes partial slot w + b,
// unique because the ranges are ordered.  seg_first[b] / seg_last[b] record the first
// and last range touching request b; info[0] records W.
//
// kSegmentCost is what a segment's fixed work costs in 32-token tiles, kSegmentCostT8 the
// same for the FP8 formats in their 64-token tiles: the query load and split, the
// pipeline fill and drain, and the partial store.  Measured per workgroup (cycles or end
// time against tiles and segments over the 256 ranges of the B=64, H=128 FP8 workload):
// about 50700 cycles (24-26 us) per segment against about 6550 cycles per 64-token tile,
// i.e. 8 tiles; the 32-token figure (17 us against 1.6 us per tile) is from the
// 32-token loop with NVFP4 dequantisation.
// An empty range can only sit where one request ends and the next begins, so every
// range between seg_first[b] and seg_last[b] holds tiles of b exactly when its cost
// interval is not empty (the combine relies on this).
constexpr int kSegmentCost = 10;
constexpr int kSegmentCostT8 = 8;

template <int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_paged_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<FMT>()];
  // tokens per tile (the FP8 formats stream 64-token tiles) and the per-segment cost in
  // those tiles
  constexpr bool kFp8Fmt = FMT == kFmtFp8 || FMT == kFmtFp8Q;
  constexpr int TT = kFp8Fmt ? kT8 : kTileTokens;
  constexpr int SC = kFp8Fmt ? kSegmentCostT8 : kSegmentCost;
  __shared__ int wsum[2][kWaves];
  __shared__ int found[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int max_len = p.max_blocks * p.page_size;
  // with a window, a request's tiles start at the one holding its first visible token
  // (query 0 at position n - q_len sees from n - q_len - window + 1)
  auto first_tile = [&](int n) { return p.window > 0 ? max(n - p.q_len - p.window + 1, 0) / TT : 0; };
  auto tiles_of = [&](int b) {
    const int n = min(max(p.seq_lens[b], 0), max_len);
    return n > 0 ? (n + TT - 1) / TT - first_tile(n) : 0;
  };

  // workgroup id -> (range w, row group rg).  Ids are dealt round-robin over the 8 XCDs;
  // XCD x takes the consecutive ranges x * per_xcd .. x * per_xcd + per_xcd - 1 with all
  // their row groups, so the neighbouring ranges of one request (and its query) share
  // that XCD's L2.  The grid holds 8 * per_xcd * row_groups ids.
  const int id = blockIdx.x;
  const int per_xcd = (p.num_splits + 7) / 8, k = id / 8;
  const int rg = k % p.row_groups;
  const int w = (id % 8) * per_xcd + k / p.row_groups;
  if (w >= p.num_splits) return;

  // tile counts and costs: thread t sums requests [s0, s1); exclusive scans give each
  // chunk's first tile and first cost position, and the totals T and W
  auto cost_of = [](int nb) { return nb > 0 ? nb + SC : 0; };
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;  // an empty range unless set below
  const int per = (p.B + kThreads - 1) / kThreads;
  const int s0 = min(tid * per, p.B), s1 = min(s0 + per, p.B);
  int acc = 0, accc = 0;
  for (int b = s0; b < s1; ++b) {
    const int nb = tiles_of(b);
    acc += nb;
    accc += cost_of(nb);
  }
  int x = acc, xc = accc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o), yc = __shfl_up(xc, o);
    if (lane >= o) x += y, xc += yc;
  }
  if (lane == 63) wsum[0][wave] = x, wsum[1][wave] = xc;
  __syncthreads();
  int start = x - acc, cstart = xc - accc, T = 0, W = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    start += (i < wave) ? wsum[0][i] : 0;
    cstart += (i < wave) ? wsum[1][i] : 0;
    T += wsum[0][i];
    W += wsum[1][i];
  }
  if (w == 0 && rg == 0 && tid == 0) p.info[0] = W;
  if (W == 0) return;  // uniform: no tiles at all
  // cost position c in [0, W) -> the request whose cost span holds it, that request's
  // first tile, and the tile c maps to; the thread whose chunk holds c walks its requests
  const int64_t lo = ((int64_t)w * W) / p.num_splits, hi = ((int64_t)(w + 1) * W) / p.num_splits;
  auto locate = [&](int64_t c, int& req, int& first, int& tile) {
    int64_t cb = cstart;
    int tb = start;
    for (int b = s0; b < s1; ++b) {
      const int nb = tiles_of(b);
      if (c < cb + cost_of(nb)) {
        req = b;
        first = tb;
        tile = tb + (int)max(c - cb - SC, (int64_t)0);
        return;
      }
      cb += cost_of(nb);
      tb += nb;
    }
  };
  if (cstart <= lo && lo < cstart + accc) locate(lo, found[0], found[1], found[2]);  // exactly one thread
  if (hi >= W) {  // the last range ends with the batch
    if (tid == 0) found[3] = T;
  } else if (cstart <= hi && hi < cstart + accc) {
    int req, first;
    locate(hi, req, first, found[3]);
  }
  __syncthreads();
  const int t0 = found[2], t1 = found[3];
  if (t0 >= t1) return;  // uniform over the workgroup
  int b = found[0], base = found[1];
  int t = t0;
  while (t < t1) {
    const int nb = tiles_of(b);
    if (base + nb <= t) {  // empty request
      base += nb;
      ++b;
      continue;
    }
    const int seg_end = min(t1, base + nb);
    const int n = min(max(p.seq_lens[b], 0), max_len);
    const int tf = first_tile(n);  // run_range counts tiles from the request's token 0
    // these are the same in every lane (read from LDS words and tables that all lanes
    // share); saying so keeps the page addresses in scalar registers
    auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    if constexpr (kFp8Fmt)
      run_range_fp8<FMT == kFmtFp8Q>(p, lds_addr((lds_ptr)smem), uni(b), uni(n), rg, uni(t - base + tf),
                                      uni(seg_end - base + tf), (int64_t)w + uni(b));
    else
      run_range<FMT, true>(p, lds_addr((lds_ptr)smem), uni(b), uni(n), rg, uni(t - base + tf),
                           uni(seg_end - base + tf), (int64_t)w + uni(b));
    if (tid == 0 && rg == 0) {
      if (t == base) p.seg_first[b] = w;
      if (seg_end == base + nb) p.seg_last[b] = w;
    }
    t = seg_end;
    base += nb;
    ++b;
  }
}

// Paged, fixed-length splits (the pages' own split form): U = row_groups * max_splits * B
// work items (row group, split j, request b), dealt to the XCDs in consecutive blocks as
// in the contiguous kernel (a request's splits share one L2); split j of request b
// covers tokens [j L, min((j + 1) L, n_b)), L = kv_len_per_split
// (a power of two >= 128, so a whole number of tiles of either size), and writes slot
// b * rows * NS + j of o_part [B, rows, NS, 512] / lse_part [B, rows, NS].  A split past
// the request's end writes lse = -inf for its rows and leaves its O_j, which the combine
// then weighs 0, unwritten.
template <int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_paged_splits_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<FMT>()];
  constexpr bool kFp8Fmt = FMT == kFmtFp8 || FMT == kFmtFp8Q;
  constexpr int TT = kFp8Fmt ? kT8 : kTileTokens;
  const int64_t U = (int64_t)p.row_groups * p.num_splits * p.B, per = (U + 7) / 8;
  const int64_t u = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (u >= U) return;
  const int rg = (int)(u % p.row_groups), j = (int)((u / p.row_groups) % p.num_splits);
  const int b = (int)(u / ((int64_t)p.row_groups * p.num_splits));
  const int n = min(max(p.seq_lens[b], 0), p.max_blocks * p.page_size);
  const int t0 = j * p.kv_len_per_split, t1 = min(t0 + p.kv_len_per_split, n);
  const int64_t slot = (int64_t)b * p.rows * p.num_splits + j;
  if (t0 >= t1) {  // uniform over the workgroup
    const int row = rg * kRowsPerGroup + (int)threadIdx.x;
    if ((int)threadIdx.x < kRowsPerGroup && row < p.rows) p.lse_part[slot * p.l_slot + (int64_t)row * p.l_row] = -INFINITY;
    return;
  }
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  if constexpr (kFp8Fmt)
    run_range_fp8<FMT == kFmtFp8Q>(p, lds_addr((lds_ptr)smem), uni(b), uni(n), rg, uni(t0 / TT),
                                    uni((t1 + TT - 1) / TT), slot);
  else
    run_range<FMT, true>(p, lds_addr((lds_ptr)smem), uni(b), uni(n), rg, uni(t0 / TT), uni((t1 + TT - 1) / TT),
                         slot);
}

// ------------------------------------------------------------------------------------
// combine kernels (one wavefront per output row)
// ------------------------------------------------------------------------------------

// Merge ns partials of one row; lse(j) returns lse_j (-inf for an empty or dead split)
// and opart(j) the address of O_j.  sink: an extra logit of the row that joins the
// denominator and carries no value (-inf: none).  Lane j % 64 holds lse_j, so the row's
// maximum, LSE and weights take wavefront reductions instead of a serial walk.  Up to 8
// partials (the usual case), every O_j load goes out together with the lse loads, since
// their addresses do not depend on the weights: one memory round trip instead of two.
// Beyond that the O_j loads go out four splits at a time after the weights.  An O_j of
// weight 0 (lse_j = -inf, or too far below the row's LSE) is loaded but adds nothing, NaN
// included.
template <class Lse, class OPart>
__device__ __forceinline__ void combine_row(int ns, Lse lse, OPart opart, uint16_t* orow, float* lse_out, int lane,
                                            float sink = -INFINITY) {
  auto store = [&](const float* acc, float LSE) {  // bf16 O (nearest even) and the row's LSE
    u32x4 packed;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      packed[i] = (unsigned)f32_to_bf16_rne(acc[2 * i]) | ((unsigned)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4*>(orow + 8 * lane) = packed;
    if (lse_out && lane == 0) *lse_out = LSE;
  };
  constexpr int kPre = 8;
  f32x4 pa[kPre], pb[kPre];
  if (ns <= kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (u < ns) {
        const f32x4* src = reinterpret_cast<const f32x4*>(opart(u) + 8 * lane);
        pa[u] = src[0];
        pb[u] = src[1];
      }
  }
  const float l0 = lane < ns ? lse(lane) : -INFINITY;  // the first 64 splits' lse, read once
  if (ns <= kPre) {
    float M = fmaxf(wave_max(l0), sink);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float LSE = -INFINITY;
    if (M != -INFINITY) {
      const float den = wave_sum(expf(l0 - M)) + (sink != -INFINITY ? expf(sink - M) : 0.f);
      LSE = M + logf(den);
      const float wl = expf(l0 - LSE);
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        if (u < ns) {
          const float wgt = __shfl(wl, u);
          const bool on = wgt != 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] += on ? wgt * pa[u][e] : 0.f;
            acc[4 + e] += on ? wgt * pb[u][e] : 0.f;
          }
        }
      }
    }
    store(acc, LSE);
    return;
  }
  float M = l0;
  for (int j = lane + 64; j < ns; j += 64) M = fmaxf(M, lse(j));
  M = fmaxf(wave_max(M), sink);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float LSE = -INFINITY;
  if (M != -INFINITY) {
    float den = expf(l0 - M);
    for (int j = lane + 64; j < ns; j += 64) den += expf(lse(j) - M);
    den = wave_sum(den) + (sink != -INFINITY ? expf(sink - M) : 0.f);
    LSE = M + logf(den);
    for (int j0 = 0; j0 < ns; j0 += 64) {
      const int nc = min(ns - j0, 64);
      const float lj = j0 == 0 ? l0 : (lane < nc ? lse(j0 + lane) : -INFINITY);
      const float wl = expf(lj - LSE);  // weight of split j0 + lane
      constexpr int kBatch = 4;
      for (int jb = 0; jb < nc; jb += kBatch) {
        f32x4 a[kBatch], b[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (jb + u < nc) {
            const f32x4* src = reinterpret_cast<const f32x4*>(opart(j0 + jb + u) + 8 * lane);
            a[u] = src[0];
            b[u] = src[1];
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (jb + u < nc) {
            const float wgt = __shfl(wl, jb + u);
            const bool on = wgt != 0.f;  // a weight-0 split adds nothing, whatever its O_j holds
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[e] += on ? wgt * a[u][e] : 0.f;
              acc[4 + e] += on ? wgt * b[u][e] : 0.f;
            }
          }
        }
      }
    }
  }
  store(acc, LSE);
}

// generic: o_part [rows, ns, 512], lse_part [rows, ns]
__global__ __launch_bounds__(256) void combine_generic_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const float* lses = p.lse_part + row * p.num_splits;
  const float* base = p.o_part + row * p.num_splits * kLatent;
  auto lse = [&](int j) { return lses[j]; };
  auto opart = [&](int j) { return base + (int64_t)j * kLatent; };
  combine_row(p.num_splits, lse, opart, p.o + row * kLatent, p.lse ? p.lse + row : nullptr, lane);
}

// Many partials of one row (more than 8): one workgroup of kCW wavefronts per row.
// Wavefront w merges the partials j = w, w + kCW, .. on its own (O_j loads issued with the
// lse loads, up to 8 per round trip) relative to its own maximum M_w; the kCW results
// (M_w, D_w = sum of exp(lse_j - M_w), A_w = sum of exp(lse_j - M_w) O_j) are then merged
// through the LDS: with M = max M_w, O = sum of exp(M_w - M) A_w / D and LSE = M + log D,
// D = sum of exp(M_w - M) D_w (+ exp(sink - M)).  A row with hundreds of partials takes
// a few round trips instead of one per four partials.
constexpr int kCW = 8;  // wavefronts per row
template <class Lse, class OPart>
__device__ __forceinline__ void combine_row_wide(int ns, Lse lse, OPart opart, uint16_t* orow, float* lse_out,
                                                 float sink = -INFINITY) {
  __shared__ float xm[kCW], xd[kCW];
  __shared__ f32x4 xa[kCW][2][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int kB = 8;
  float Mw = -INFINITY, Dw = 0.f;
  f32x4 aw = {0.f, 0.f, 0.f, 0.f}, bw = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = w; j0 < ns; j0 += kCW * kB) {  // this wavefront's partials j0, j0 + kCW, .. (up to kB)
    f32x4 a[kB], b[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = j0 + kCW * u;
      if (j < ns) {
        const f32x4* src = reinterpret_cast<const f32x4*>(opart(j) + 8 * lane);
        a[u] = src[0];
        b[u] = src[1];
      }
    }
    const float l = (lane < kB && j0 + kCW * lane < ns) ? lse(j0 + kCW * lane) : -INFINITY;
    const float Mn = fmaxf(Mw, wave_max(l));
    if (Mn == -INFINITY) continue;  // nothing seen yet (uniform)
    const float r = Mw == -INFINITY ? 0.f : expf(Mw - Mn);  // rescale what came before
    const float e = expf(l - Mn);
    Dw = Dw * r + wave_sum(e);
    aw *= r;
    bw *= r;
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (j0 + kCW * u < ns) {
        const float wgt = __shfl(e, u);
        if (wgt != 0.f) {  // a weight-0 partial adds nothing, whatever its O_j holds
          aw += wgt * a[u];
          bw += wgt * b[u];
        }
      }
    }
    Mw = Mn;
  }
  if (lane == 0) {
    xm[w] = Mw;
    xd[w] = Dw;
  }
  xa[w][0][lane] = aw;
  xa[w][1][lane] = bw;
  __syncthreads();
  if (w != 0) return;
  float M = sink;
#pragma unroll
  for (int v = 0; v < kCW; ++v) M = fmaxf(M, xm[v]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float LSE = -INFINITY;
  if (M != -INFINITY) {
    float D = sink != -INFINITY ? expf(sink - M) : 0.f, s[kCW];
#pragma unroll
    for (int v = 0; v < kCW; ++v) {
      s[v] = xm[v] == -INFINITY ? 0.f : expf(xm[v] - M);
      D += s[v] * xd[v];
    }
    LSE = M + logf(D);
    const float inv = 1.f / D;
#pragma unroll
    for (int v = 0; v < kCW; ++v) {
      const f32x4 ta = xa[v][0][lane], tb = xa[v][1][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += s[v] * ta[e];
        acc[4 + e] += s[v] * tb[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }
  u32x4 packed;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    packed[i] = (unsigned)f32_to_bf16_rne(acc[2 * i]) | ((unsigned)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(orow + 8 * lane) = packed;
  if (lse_out && lane == 0) *lse_out = LSE;
}

// generic, more than 8 partials per row: one workgroup per row
__global__ __launch_bounds__(64 * kCW) void combine_generic_wide_kernel(const CombineParams p) {
  const int64_t row = blockIdx.x;
  const int ns = p.num_splits;
  const float* lses = p.lse_part + row * ns;
  const float* base = p.o_part + row * ns * kLatent;
  combine_row_wide(ns, [&](int j) { return lses[j]; }, [&](int j) { return base + (int64_t)j * kLatent; },
                   p.o + row * kLatent, p.lse ? p.lse + row : nullptr);
}

// paged: row (b, r) merges slots w + b for the non-empty ranges w in
// [seg_first[b], seg_last[b]]; o_part [slots, rows, 512], lse_part [slots, rows]
// The partials of paged row grow (request b, row r): the ranges w0 .. w1 that touch b.
struct PagedRow {
  const CombineParams* p;
  int b, r, w0, w1, W;
  __device__ PagedRow(const CombineParams& c, int64_t grow) : p(&c) {
    b = (int)(grow / c.rows);
    r = (int)(grow % c.rows);
    const int n = min(max(c.seq_lens[b], 0), c.max_len);
    W = c.info[0];  // total cost of the batch's ranges (see decode_paged_kernel)
    const int G = c.num_splits;
    w0 = 0;
    w1 = -1;
    if (n > 0) {  // descriptors written by the decode launch; clamped so they never address outside
      w0 = min(max(c.seg_first[b], 0), G - 1);
      w1 = min(max(c.seg_last[b], w0), G - 1);
    }
  }
  // a dead range (no tiles) wrote nothing: its lse counts as -inf (its slot is still
  // inside the workspace, so the unused load of its O_j stays in bounds)
  __device__ bool live(int wj) const {
    const int G = p->num_splits;
    return ((int64_t)wj * W) / G < ((int64_t)(wj + 1) * W) / G;  // range wj holds tiles
  }
  __device__ float lse(int j) const {
    const int wj = w0 + j;
    return live(wj) ? p->lse_part[((int64_t)wj + b) * p->rows + r] : -INFINITY;
  }
  __device__ const float* opart(int j) const { return p->o_part + (((int64_t)w0 + j + b) * p->rows + r) * kLatent; }
  __device__ float sink() const { return p->sinks ? p->sinks[r % p->H] : -INFINITY; }
};

// paged: row (b, r) merges slots w + b for the non-empty ranges w in
// [seg_first[b], seg_last[b]]; o_part [slots, rows, 512], lse_part [slots, rows].  One
// wavefront per row.
__global__ __launch_bounds__(256) void combine_paged_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grow >= (int64_t)p.B * p.rows) return;
  const PagedRow R(p, grow);
  combine_row(R.w1 - R.w0 + 1, [&](int j) { return R.lse(j); }, [&](int j) { return R.opart(j); },
              p.o + grow * kLatent, p.lse ? p.lse + grow : nullptr, lane, R.sink());
}

// paged, with requests spread over many ranges: one workgroup per row (combine_row_wide)
__global__ __launch_bounds__(64 * kCW) void combine_paged_wide_kernel(const CombineParams p) {
  const int64_t grow = blockIdx.x;
  const PagedRow R(p, grow);
  combine_row_wide(R.w1 - R.w0 + 1, [&](int j) { return R.lse(j); }, [&](int j) { return R.opart(j); },
                   p.o + grow * kLatent, p.lse ? p.lse + grow : nullptr, R.sink());
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------

// Few heads: the wavefronts of a row block share its output dims (D = 4 up to 32 rows,
// 2 up to 64) instead of repeating its last row.
hipError_t launch_decode_contig(const DecodeParams& p, hipStream_t stream) {
  const int D = p.rows <= kWaveRows ? 4 : p.rows <= 2 * kWaveRows ? 2 : 1;
  // row_groups counts groups of 128 / D rows (checked by the caller against the grid's
  // size limit)
  const int U = p.row_groups * p.num_splits * p.B;
  const dim3 grid((unsigned)(((U + 7) / 8) * 8));
  if (D == 4) hipLaunchKernelGGL(decode_contig_kernel<4>, grid, dim3(kThreads), 0, stream, p);
  else if (D == 2) hipLaunchKernelGGL(decode_contig_kernel<2>, grid, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(decode_contig_kernel<1>, grid, dim3(kThreads), 0, stream, p);
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
      hipLaunchKernelGGL(decode_paged_kernel<kFmtFp8Q>, dim3(blocks), dim3(kThreads), 0, stream, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_paged_splits(int fmt, const DecodeParams& p, hipStream_t stream) {
  const int64_t U = (int64_t)p.row_groups * p.num_splits * p.B;
  const dim3 grid((unsigned)(((U + 7) / 8) * 8));
  switch (fmt) {
    case kFmtBf16:
      hipLaunchKernelGGL(decode_paged_splits_kernel<kFmtBf16>, grid, dim3(kThreads), 0, stream, p);
      break;
    case kFmtFp8:
      hipLaunchKernelGGL(decode_paged_splits_kernel<kFmtFp8>, grid, dim3(kThreads), 0, stream, p);
      break;
    case kFmtNvfp4:
      hipLaunchKernelGGL(decode_paged_splits_kernel<kFmtNvfp4>, grid, dim3(kThreads), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL(decode_paged_splits_kernel<kFmtFp8Q>, grid, dim3(kThreads), 0, stream, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_generic(const CombineParams& p, hipStream_t stream) {
  if (p.num_splits > 8)
    hipLaunchKernelGGL(combine_generic_wide_kernel, dim3((unsigned)p.rows), dim3(64 * kCW), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_generic_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// A request spans about num_splits / B ranges; beyond 16 on average its rows take a
// workgroup each.
hipError_t launch_combine_paged(const CombineParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.rows;
  if (p.num_splits > 16 * p.B)
    hipLaunchKernelGGL(combine_paged_wide_kernel, dim3((unsigned)rows), dim3(64 * kCW), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_paged_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
