// C ABI of libmla_decode.so (declared in include/mla_decode.h): argument checks, the
// split planners, workspace layout and kernel launches.  No allocation, no
// synchronisation, no device reads on the host.

#include "mla_decode.h"
#include "mla_internal.h"

#include <math.h>
#include <stdint.h>

namespace {

using namespace mla;

constexpr float kLog2e = 1.44269504088896341f;

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int64_t next_pow2(int64_t n) {
  // smallest power of two >= n, 1 for n <= 0 (TileGym page, helper next_power_of_2)
  if (n <= 0) return 1;
  int64_t p = 1;
  while (p < n) p <<= 1;
  return p;
}

int64_t row_bytes(int fmt) {
  switch (fmt) {
    case MLA_KV_BF16: return 2 * kRow;
    case MLA_KV_FP8_E4M3:
    case MLA_KV_FP8_E4M3_QFP8: return kRow;
    case MLA_KV_NVFP4: return kRow / 2 + kRow / 16;
    default: return -1;
  }
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PagedLayout {
  size_t o_off, lse_off, first_off, last_off, info_off, total;
  int64_t slots;
};

// fixed-length paged splits: o_part [B][rows][NS][512] f32 | lse_part [B][rows][NS] f32,
// the second section 256-byte aligned
struct SplitsLayout {
  size_t lse_off, total;
};
bool splits_layout(int B, int q_len, int H, int max_splits, SplitsLayout* L) {
  if (B < 1 || B > MLA_MAX_BATCH || q_len < 1 || q_len > MLA_MAX_Q_LEN || H < 16 || H > MLA_MAX_HEADS ||
      H % 16 != 0 || max_splits < 1 || max_splits > 65535)
    return false;
  const int64_t n = (int64_t)B * q_len * H * max_splits;
  L->lse_off = round_up((size_t)(n * kLatent * 4), 256);
  L->total = L->lse_off + round_up((size_t)(n * 4), 256);
  return true;
}

// workspace: o_part [slots][rows][512] f32 | lse_part [slots][rows] f32 | first [B] i32 |
// last [B] i32 | info [64] i32, each section 256-byte aligned
bool paged_layout(int B, int q_len, int H, int num_splits, PagedLayout* L) {
  if (B < 1 || B > MLA_MAX_BATCH || q_len < 1 || q_len > MLA_MAX_Q_LEN || H < 16 || H > MLA_MAX_HEADS ||
      H % 16 != 0 || num_splits < 1 || num_splits > MLA_MAX_SPLITS)
    return false;
  const int64_t rows = (int64_t)q_len * H;
  L->slots = (int64_t)num_splits + B - 1;
  L->o_off = 0;
  L->lse_off = round_up((size_t)(L->slots * rows * kLatent * 4), 256);
  L->first_off = L->lse_off + round_up((size_t)(L->slots * rows * 4), 256);
  L->last_off = L->first_off + round_up((size_t)B * 4, 256);
  L->info_off = L->last_off + round_up((size_t)B * 4, 256);
  L->total = L->info_off + 256;
  return true;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: configuration not supported";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: workspace below mla_paged_workspace_bytes";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: kernel launch failed";
    case MLA_ERR_SCRATCH_LIMIT:
      return "MLA_ERR_SCRATCH_LIMIT: the problem's workspace exceeds the built-in scratch (MLA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown mla_status";
  }
}

int mla_device_num_cus(int device, int* num_cus) {
  if (!num_cus) return MLA_ERR_INVALID_ARG;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v <= 0)
    return MLA_ERR_HIP;
  *num_cus = v;
  return MLA_OK;
}

int mla_plan_contig(int num_cus, int B, int S_kv, int* kv_len_per_split, int* num_splits) {
  if (!kv_len_per_split || !num_splits || num_cus < 1 || B < 1 || S_kv < 1) return MLA_ERR_INVALID_ARG;
  // TileGym page, _mla_decoding_split_kv.forward
  const int est = num_cus / B > 1 ? num_cus / B : 1;
  int64_t L = next_pow2(S_kv / est);
  if (L < 128) L = 128;
  *kv_len_per_split = (int)L;
  *num_splits = (int)((S_kv + L - 1) / L);
  return MLA_OK;
}

int mla_plan_paged(int num_cus, int B, int q_len, int H, int* num_splits) {
  if (!num_splits || num_cus < 1 || B < 1 || q_len < 1 || H < 1) return MLA_ERR_INVALID_ARG;
  const int64_t groups = ((int64_t)q_len * H + kRowsPerGroup - 1) / kRowsPerGroup;
  int64_t g = num_cus / groups;
  if (g < 1) g = 1;
  if (g > MLA_MAX_SPLITS) g = MLA_MAX_SPLITS;
  *num_splits = (int)g;
  return MLA_OK;
}

size_t mla_paged_workspace_bytes(int B, int q_len, int H, int num_splits) {
  PagedLayout L;
  if (!paged_layout(B, q_len, H, num_splits, &L)) return 0;
  return L.total;
}

int mla_decode_splitkv(const uint16_t* q, const uint16_t* qpe, const uint16_t* kv, const uint16_t* kpe, int B,
                       int H, int S_kv, float sm_scale, int kv_len_per_split, float* o_part, float* lse_part,
                       void* stream) {
  if (!q || !qpe || !kv || !kpe || !o_part || !lse_part) return MLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(qpe, 16) || !aligned(kv, 16) || !aligned(kpe, 16) || !aligned(o_part, 16) ||
      !aligned(lse_part, 4))
    return MLA_ERR_INVALID_ARG;
  if (B < 1 || S_kv < 1 || !isfinite(sm_scale) || sm_scale < 0.f) return MLA_ERR_INVALID_ARG;
  if (H < 16 || H > MLA_MAX_HEADS || H % 16 != 0) return MLA_ERR_UNSUPPORTED;
  // the page's assertions: power of two and at least TILE_N = 128
  if (kv_len_per_split < 128 || (kv_len_per_split & (kv_len_per_split - 1)) != 0) return MLA_ERR_INVALID_ARG;
  const int ns = (S_kv + kv_len_per_split - 1) / kv_len_per_split;
  // one workgroup per (request, split): the count must fit the kernel's int indexing
  if (ns > 65535 || B > 65535 || (int64_t)ns * B > (int64_t)(1 << 30)) return MLA_ERR_INVALID_ARG;

  DecodeParams p{};
  p.q = q;
  p.qpe = qpe;
  p.kv = kv;
  p.kpe = kpe;
  p.S = S_kv;
  p.kv_len_per_split = kv_len_per_split;
  p.B = B;
  p.q_len = 1;
  p.H = H;
  p.rows = H;
  p.row_groups = 1;  // H <= 128 rows: one group (of 128 / D rows for few heads)
  p.num_splits = ns;
  p.score_scale = sm_scale * kLog2e;
  p.v_scale = 1.f;
  p.o_part = o_part;
  p.lse_part = lse_part;
  // element (b, h, j) of o_part [B, H, NS, 512] sits at ((b*H + h)*NS + j)*512: the
  // kernel addresses slot*o_slot + row*o_row with slot = b*H*NS + j and row = h.
  p.o_slot = kLatent;
  p.o_row = (int64_t)ns * kLatent;
  p.l_slot = 1;
  p.l_row = ns;
  if (launch_decode_contig(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_splitkv_combine(const float* o_part, const float* lse_part, int rows, int num_splits, uint16_t* o,
                        float* lse, void* stream) {
  if (!o_part || !lse_part || !o) return MLA_ERR_INVALID_ARG;
  if (!aligned(o_part, 16) || !aligned(lse_part, 4) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
    return MLA_ERR_INVALID_ARG;
  if (rows < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_INVALID_ARG;
  CombineParams c{};
  c.o_part = o_part;
  c.lse_part = lse_part;
  c.o = o;
  c.lse = lse;
  c.rows = rows;
  c.num_splits = num_splits;
  if (launch_combine_generic(c, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"

namespace {

// Host checks shared by the paged entry points.
int check_paged_shape(int B, int q_len, int H, int num_splits, const void* workspace, size_t workspace_bytes,
                      PagedLayout* L) {
  if (!workspace || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (H < 16 || H > MLA_MAX_HEADS || H % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (B < 1 || B > MLA_MAX_BATCH) return MLA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_INVALID_ARG;
  if (!paged_layout(B, q_len, H, num_splits, L)) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < L->total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  return MLA_OK;
}

// Checks of the cache, table and scale arguments shared by the paged decodes.
int check_paged_cache(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                      int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* seq_lens, int B, float sm_scale) {
  if (!q || !qpe || !kv_cache || !block_tables || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(qpe, 16) || !aligned(kv_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4))
    return MLA_ERR_INVALID_ARG;
  const int64_t rb = row_bytes(fmt);
  if (rb < 0) return MLA_ERR_UNSUPPORTED;
  if (page_size != 32 && page_size != 64) return MLA_ERR_UNSUPPORTED;
  if (num_pages < 1 || max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (page_stride_bytes < page_size * rb || page_stride_bytes % 16 != 0) return MLA_ERR_INVALID_ARG;
  if ((int64_t)B * max_blocks_per_seq * page_size >= ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARG;
  if (!isfinite(sm_scale) || sm_scale < 0.f) return MLA_ERR_INVALID_ARG;
  const bool fp8 = (fmt == MLA_KV_FP8_E4M3 || fmt == MLA_KV_FP8_E4M3_QFP8);
  if (fp8 && !(isfinite(kv_scale) && kv_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// The paged decode's parameters that do not depend on the split form.
DecodeParams paged_params(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                          int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                          int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H, float sm_scale) {
  const bool fp8 = (fmt == MLA_KV_FP8_E4M3 || fmt == MLA_KV_FP8_E4M3_QFP8);
  const float vs = fp8 ? kv_scale : 1.f;
  DecodeParams p{};
  p.q = q;
  p.qpe = qpe;
  p.cache = static_cast<const uint8_t*>(kv_cache);
  p.page_stride = page_stride_bytes;
  p.block_tables = block_tables;
  p.max_blocks = max_blocks_per_seq;
  p.seq_lens = seq_lens;
  p.page_size = page_size;
  p.page_shift = page_size == 64 ? 6 : 5;
  p.num_pages = num_pages;
  p.B = B;
  p.q_len = q_len;
  p.H = H;
  p.rows = q_len * H;
  p.row_groups = (p.rows + kRowsPerGroup - 1) / kRowsPerGroup;
  p.score_scale = sm_scale * vs * kLog2e;
  p.v_scale = vs;
  return p;
}

int paged_partials(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                   int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                   int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                   int window, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 0) return MLA_ERR_INVALID_ARG;
  int st = check_paged_cache(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                             max_blocks_per_seq, seq_lens, B, sm_scale);
  if (st != MLA_OK) return st;
  PagedLayout L;
  st = check_paged_shape(B, q_len, H, num_splits, workspace, workspace_bytes, &L);
  if (st != MLA_OK) return st;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  DecodeParams p = paged_params(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes,
                                block_tables, max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale);
  p.num_splits = num_splits;
  p.window = window;
  p.o_part = reinterpret_cast<float*>(ws + L.o_off);
  p.lse_part = reinterpret_cast<float*>(ws + L.lse_off);
  p.o_slot = (int64_t)p.rows * kLatent;
  p.o_row = kLatent;
  p.l_slot = p.rows;
  p.l_row = 1;
  p.seg_first = reinterpret_cast<int32_t*>(ws + L.first_off);
  p.seg_last = reinterpret_cast<int32_t*>(ws + L.last_off);
  p.info = reinterpret_cast<int32_t*>(ws + L.info_off);
  if (launch_decode_paged(fmt, p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int paged_combine(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens, int B, int q_len, int H,
                  int num_splits, int max_blocks_per_seq, int page_size, const float* sinks, uint16_t* o,
                  float* lse, void* stream) {
  if (!seq_lens || !o || !aligned(seq_lens, 4) || !aligned(o, 16) || (lse && !aligned(lse, 4)) ||
      (sinks && !aligned(sinks, 4)))
    return MLA_ERR_INVALID_ARG;
  PagedLayout L;
  const int st = check_paged_shape(B, q_len, H, num_splits, workspace, workspace_bytes, &L);
  if (st != MLA_OK) return st;
  if (page_size != 32 && page_size != 64) return MLA_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < 1 || (int64_t)B * max_blocks_per_seq * page_size >= ((int64_t)1 << 31))
    return MLA_ERR_INVALID_ARG;
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  CombineParams c{};
  c.o_part = reinterpret_cast<const float*>(ws + L.o_off);
  c.lse_part = reinterpret_cast<const float*>(ws + L.lse_off);
  c.o = o;
  c.lse = lse;
  c.rows = q_len * H;
  c.num_splits = num_splits;
  c.B = B;
  c.seq_lens = seq_lens;
  c.seg_first = reinterpret_cast<const int32_t*>(ws + L.first_off);
  c.seg_last = reinterpret_cast<const int32_t*>(ws + L.last_off);
  c.info = reinterpret_cast<const int32_t*>(ws + L.info_off);
  c.max_len = max_blocks_per_seq * page_size;
  c.sinks = sinks;
  c.H = H;
  if (launch_combine_paged(c, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_paged_decode_partials(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                              int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H,
                              float sm_scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return paged_partials(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                        max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale, 0, num_splits, workspace,
                        workspace_bytes, stream);
}

int mla_paged_combine(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens, int B, int q_len,
                      int H, int num_splits, int max_blocks_per_seq, int page_size, uint16_t* o, float* lse,
                      void* stream) {
  return paged_combine(workspace, workspace_bytes, seq_lens, B, q_len, H, num_splits, max_blocks_per_seq, page_size,
                       nullptr, o, lse, stream);
}

int mla_paged_decode(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                     int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                     int num_splits, void* workspace, size_t workspace_bytes, uint16_t* o, float* lse,
                     void* stream) {
  return mla_paged_decode_ext(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                              max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale, 0, nullptr, num_splits, workspace,
                              workspace_bytes, o, lse, stream);
}

int mla_plan_paged_splits(int num_cus, int B, int q_len, const int32_t* seq_lens_host, int page_size,
                          int* kv_len_per_split, int* max_splits) {
  if (!seq_lens_host || !kv_len_per_split || !max_splits || num_cus < 1 || B < 1 || B > MLA_MAX_BATCH)
    return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (page_size != 32 && page_size != 64) return MLA_ERR_UNSUPPORTED;
  int64_t max_len = 1;
  for (int b = 0; b < B; ++b)
    if (seq_lens_host[b] > max_len) max_len = seq_lens_host[b];
  // TileGym page, _mla_decoding_split_kv.forward, with the batch's longest sequence as S_kv
  const int est = num_cus / B > 1 ? num_cus / B : 1;
  int64_t L = next_pow2(max_len / est);
  if (L < 128) L = 128;
  const int64_t ns = (max_len + L - 1) / L;
  if (ns > 65535) return MLA_ERR_INVALID_ARG;
  *kv_len_per_split = (int)L;
  *max_splits = (int)ns;
  return MLA_OK;
}

size_t mla_paged_splits_workspace_bytes(int B, int q_len, int H, int max_splits) {
  SplitsLayout L;
  if (!splits_layout(B, q_len, H, max_splits, &L)) return 0;
  return L.total;
}

int mla_paged_decode_splits(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                            int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                            int kv_len_per_split, int max_splits, void* workspace, size_t workspace_bytes,
                            uint16_t* o, float* lse, void* stream) {
  int st = check_paged_cache(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                             max_blocks_per_seq, seq_lens, B, sm_scale);
  if (st != MLA_OK) return st;
  if (!o || !aligned(o, 16) || (lse && !aligned(lse, 4))) return MLA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256)) return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (H < 16 || H > MLA_MAX_HEADS || H % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (B < 1 || B > MLA_MAX_BATCH) return MLA_ERR_INVALID_ARG;
  // the page's assertions on the split length; the splits must cover every admissible length
  if (kv_len_per_split < 128 || (kv_len_per_split & (kv_len_per_split - 1)) != 0) return MLA_ERR_INVALID_ARG;
  if (max_splits < 1 || max_splits > 65535) return MLA_ERR_INVALID_ARG;
  if ((int64_t)max_splits * kv_len_per_split < (int64_t)max_blocks_per_seq * page_size) return MLA_ERR_INVALID_ARG;
  SplitsLayout W;
  if (!splits_layout(B, q_len, H, max_splits, &W)) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < W.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  DecodeParams p = paged_params(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes,
                                block_tables, max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale);
  p.kv_len_per_split = kv_len_per_split;
  p.num_splits = max_splits;
  p.window = 0;
  // element (b, row, j) at slot b * rows * NS + j, row stride NS (o_part [B, rows, NS, 512])
  p.o_part = reinterpret_cast<float*>(ws);
  p.lse_part = reinterpret_cast<float*>(ws + W.lse_off);
  p.o_slot = kLatent;
  p.o_row = (int64_t)max_splits * kLatent;
  p.l_slot = 1;
  p.l_row = max_splits;
  if (launch_decode_paged_splits(fmt, p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  CombineParams c{};
  c.o_part = p.o_part;
  c.lse_part = p.lse_part;
  c.o = o;
  c.lse = lse;
  c.rows = B * q_len * H;
  c.num_splits = max_splits;
  if (launch_combine_generic(c, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_paged_decode_ext(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt, float kv_scale,
                         int num_pages, int page_size, int64_t page_stride_bytes, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                         int sliding_window, const float* sinks, int num_splits, void* workspace,
                         size_t workspace_bytes, uint16_t* o, float* lse, void* stream) {
  // the combine's own checks (beyond the decode's) are made before either launch is enqueued
  if (!o || !aligned(o, 16) || (lse && !aligned(lse, 4)) || (sinks && !aligned(sinks, 4)))
    return MLA_ERR_INVALID_ARG;
  int st = paged_partials(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                          max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale, sliding_window, num_splits, workspace,
                          workspace_bytes, stream);
  if (st != MLA_OK) return st;
  return paged_combine(workspace, workspace_bytes, seq_lens, B, q_len, H, num_splits, max_blocks_per_seq, page_size,
                       sinks, o, lse, stream);
}

}  // extern "C"

extern "C" {

int mla_kv_append(const uint16_t* latent, const uint16_t* rope, const int32_t* slots, int T, void* kv_cache,
                  int fmt, float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes, void* stream) {
  if (T < 0) return MLA_ERR_INVALID_ARG;
  const int64_t rb = row_bytes(fmt);
  if (rb < 0) return MLA_ERR_UNSUPPORTED;
  if (page_size != 32 && page_size != 64) return MLA_ERR_UNSUPPORTED;
  if (num_pages < 1 || (int64_t)num_pages * page_size >= ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARG;
  if (page_stride_bytes < page_size * rb || page_stride_bytes % 16 != 0) return MLA_ERR_INVALID_ARG;
  const bool fp8 = (fmt == MLA_KV_FP8_E4M3 || fmt == MLA_KV_FP8_E4M3_QFP8);  // same page bytes
  if (fp8 && !(isfinite(kv_scale) && kv_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!latent || !rope || !slots || !kv_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(slots, 4) || !aligned(kv_cache, 16))
    return MLA_ERR_INVALID_ARG;
  AppendParams p{};
  p.latent = latent;
  p.rope = rope;
  p.slots = slots;
  p.cache = static_cast<uint8_t*>(kv_cache);
  p.page_stride = page_stride_bytes;
  p.T = T;
  p.page_size = page_size;
  p.num_pages = num_pages;
  p.fmt = fp8 ? kFmtFp8 : fmt;
  p.kv_scale = fp8 ? kv_scale : 1.f;
  if (launch_kv_append(p, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
