// Internal interface between the C-ABI host code (mla_api.cpp) and the gfx950 kernels
// (mla_kernels.hip: decode and combine; mla_append.hip: cache append).  Not installed;
// the public interface is include/mla_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatent = 512;  // latent width (V aliases it)
constexpr int kRope = 64;     // rope key width
constexpr int kRow = 576;     // one cache token

constexpr int kTileTokens = 32;    // tokens per KV tile streamed through LDS
constexpr int kWaves = 4;          // wavefronts per workgroup (one per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = 32;      // query rows one wavefront owns
constexpr int kRowsPerGroup = kWaveRows * kWaves;  // query rows (query x head) per workgroup: 128

constexpr int kFmtBf16 = 0;
constexpr int kFmtFp8 = 1;   // FP8 cache: query and softmax weights split into two E4M3 operands each
constexpr int kFmtNvfp4 = 2;
constexpr int kFmtFp8Q = 3;  // FP8 cache, query rounded to E4M3, score product on FP8 MFMA

// Everything one decode launch needs; passed by value as the kernel argument.
struct DecodeParams {
  const uint16_t* q;    // [B, q_len, H, 512] bf16 bits
  const uint16_t* qpe;  // [B, q_len, H, 64]
  // contiguous cache
  const uint16_t* kv;   // [B, S, 512]
  const uint16_t* kpe;  // [B, S, 64]
  int S;
  int kv_len_per_split;
  // paged cache
  const uint8_t* cache;
  int64_t page_stride;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  int page_size;
  int page_shift;       // log2(page_size)
  int num_pages;
  // problem
  int B, q_len, H;
  int rows;           // q_len * H
  int row_groups;     // ceil(rows / kRowsPerGroup)
  int num_splits;     // contiguous and fixed-split paged: splits per request; paged: token-balanced ranges
  int window;         // paged: query at position p sees tokens p - window + 1 .. p (0: all)
  float score_scale;  // sm_scale * kv_scale * log2(e)
  float v_scale;      // kv_scale (FP8) or 1
  // partial outputs: element (slot, row, d) at o_part[slot*o_slot + row*o_row + d]
  float* o_part;
  float* lse_part;
  int64_t o_slot, o_row, l_slot, l_row;
  int32_t* seg_first;  // paged: first / last range index that covers request b
  int32_t* seg_last;
  int32_t* info;       // paged: info[0] = total cost of the batch's ranges (tiles + per-request overhead)
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  uint16_t* o;
  float* lse;
  int rows;        // generic: total rows; paged: rows per request (q_len * H)
  int num_splits;  // generic: splits per row; paged: token-balanced ranges
  int B;           // paged only
  const int32_t* seq_lens;
  const int32_t* seg_first;
  const int32_t* seg_last;
  const int32_t* info;
  int max_len;     // paged: max_blocks * page_size (clamp for seq_lens)
  const float* sinks;  // paged: per-head sink logits [H] (null: none)
  int H;
};

// One cache append launch: token j's row [latent_j | rope_j] goes to flat slot slots[j].
struct AppendParams {
  const uint16_t* latent;  // [T, 512] bf16 bits
  const uint16_t* rope;    // [T, 64] bf16 bits
  const int32_t* slots;    // [T]: page * page_size + row; outside [0, num_pages * page_size): skipped
  uint8_t* cache;
  int64_t page_stride;
  int T, page_size, num_pages, fmt;
  float kv_scale;          // FP8: the stored code is that of x / kv_scale
};

hipError_t launch_decode_contig(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_paged(int fmt, const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_paged_splits(int fmt, const DecodeParams& p, hipStream_t stream);
hipError_t launch_combine_generic(const CombineParams& p, hipStream_t stream);
hipError_t launch_combine_paged(const CombineParams& p, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);

}  // namespace mla
