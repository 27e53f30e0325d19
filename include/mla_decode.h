/*
 * mla_decode.h -- C ABI of libmla_decode.so: absorbed Multi-head Latent Attention (MLA)
 * decode over a shared latent KV cache, split along the KV sequence, for AMD MI355X
 * (gfx950).
 *
 * What is computed.  Every cache token is one 576-wide row: a 512-wide latent followed
 * by a 64-wide rope key.  K and V alias the same latent (TileGym page
 * "mla_decoding_split_kv.py", _mla_decoding_split_kv.forward: "K=V=KV"; metrale page
 * "kv_cache_mla.rs", mla_paged_decode_nvfp4: 512 + 64 = 576 values per token).  For a
 * query row with latent part Q (512) and rope part QPE (64):
 *     s_t   = sm_scale * (Q . latent_t + QPE . rope_t)
 *     LSE   = log sum_t exp(s_t)                    (natural log)
 *     O     = sum_t exp(s_t - LSE) * latent_t       (512 values)
 * The token range is cut into splits; each split yields a normalised partial output
 * O_j and its log-sum-exp lse_j, and the split-K reduce merges them:
 *     LSE = log sum_j exp(lse_j);  O = sum_j exp(lse_j - LSE) * O_j
 * (TileGym page, forward: Att_Out / LSE_Out per split, then splitk_reduce).  A split a
 * row cannot see has lse_j = -inf and contributes nothing; a row that sees no token
 * gets O = 0 and LSE = -inf.
 *
 * Conventions for every entry point.
 *   - All tensor arguments are DEVICE pointers, dense and row-major, owned by the
 *     caller.  bf16 tensors are passed as their 16-bit patterns (uint16_t).  Q, QPE,
 *     KV, KPE, caches, partial outputs and outputs must be 16-byte aligned, the paged
 *     workspace 256-byte aligned, int32 tables and fp32 LSE arrays 4-byte aligned.
 *   - The library never allocates, frees, synchronises or reads device memory on the
 *     host.  Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     runs asynchronously, so the calls may be captured into a HIP graph.
 *   - Every argument is checked on the host before anything is enqueued; a failed check
 *     returns a negative mla_status and enqueues nothing.  MLA_ERR_HIP means a launch
 *     reported an error (hipGetLastError); mla_status_string names every code.
 *   - Calls on one stream are ordered; calls that share a workspace must not overlap.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Row geometry, fixed at compile time like the TileGym page's template parameters
 * (TILE_D = 512, TILE_KPE = 64). */
#define MLA_LATENT 512
#define MLA_ROPE 64
#define MLA_ROW 576

/* Limits checked on the host. */
#define MLA_MAX_HEADS 128      /* heads per call; H must be a multiple of 16 */
#define MLA_MAX_Q_LEN 8        /* query tokens per request (TokenSpeed page: q_len capacity 8) */
#define MLA_MAX_BATCH 4096     /* requests per paged call */
#define MLA_MAX_SPLITS 65536   /* num_splits of a paged call */
/* Size of the built-in workspace of mla_paged_decode_noalloc (128 MiB per GPU). */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,         /* null pointer, bad size, misalignment, bad split */
  MLA_ERR_UNSUPPORTED = -2,         /* format, page size, head count or q_len not built */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes below mla_paged_workspace_bytes */
  MLA_ERR_HIP = -4,                 /* a kernel launch failed */
  MLA_ERR_SCRATCH_LIMIT = -5        /* mla_paged_decode_noalloc: the problem needs more
                                       workspace than MLA_NOALLOC_SCRATCH_BYTES */
} mla_status;

/* Cache formats of the paged op.
 *   MLA_KV_BF16      page = [page_size][576] bf16.
 *   MLA_KV_FP8_E4M3  page = [page_size][576] OCP E4M3 ("FN") codes; value =
 *                    kv_scale * e4m3(code) for both the key and the value use
 *                    (TokenSpeed page "tokenspeed_mla.py", forward_decode: float8_e4m3fn
 *                    cache, k_scale folded into the softmax scale; metrale page,
 *                    mla_paged_decode_fp8: scalar dequant scales).
 *   MLA_KV_NVFP4     page = data [page_size][288] bytes (two E2M1 codes per byte, the
 *                    even-indexed value in the low nibble) followed by scales
 *                    [page_size][36] E4M3 bytes, scale g covering values 16g..16g+15 of
 *                    the row; value = e2m1(code) * e4m3(scale) (metrale page,
 *                    mla_paged_decode_nvfp4: packed E2M1 data followed by one E4M3 scale
 *                    per 16 values). */
typedef enum {
  MLA_KV_BF16 = 0,
  MLA_KV_FP8_E4M3 = 1,
  MLA_KV_NVFP4 = 2,
  /* Same page bytes and kv_scale as MLA_KV_FP8_E4M3, with the query rounded to E4M3
   * (nearest, ties to even, saturating at 448) and the score product on FP8 matrix cores,
   * as the TokenSpeed page's FP8 decode does (forward_decode: the query is cast to the
   * cache's FP8 type and k_scale is folded into the softmax scale).  The output product is
   * that of MLA_KV_FP8_E4M3: the softmax weights, scaled per row and 32-token tile by a
   * power of two, as two E4M3 terms (about 8 significant bits) against the raw cache codes
   * on FP8 matrix cores, with fp32 accumulation. */
  MLA_KV_FP8_E4M3_QFP8 = 3
} mla_kv_format;

/* Static text for a status code (never NULL). */
const char* mla_status_string(int status);

/* Compute units of HIP device `device` (for the planners).  Host call; does not
 * synchronise.  Returns MLA_ERR_HIP if the query fails. */
int mla_device_num_cus(int device, int* num_cus);

/* Contiguous split planner (TileGym page, _mla_decoding_split_kv.forward):
 *   estimate = max(1, num_cus / B);
 *   kv_len_per_split = max(next_power_of_2(S_kv / estimate), 128);
 *   num_splits = ceil(S_kv / kv_len_per_split).
 * Host-only integer work.  num_cus, B, S_kv >= 1. */
int mla_plan_contig(int num_cus, int B, int S_kv, int* kv_len_per_split, int* num_splits);

/* Paged split planner.  The paged op cuts the whole batch's tiles (64 tokens for the FP8
 * formats, 32 for the others) into `num_splits` contiguous ranges, one workgroup each,
 * on the device from device seq_lens (so no host copy of them is needed: the TokenSpeed
 * page avoids a device-to-host sync for the same reason, _init_prefill_metadata).  The
 * ranges are of about equal cost, where a request costs its tiles plus a fixed overhead
 * (what starting a request in a workgroup costs: query load, pipeline fill, partial
 * store) of 8 tiles for the FP8 formats and 10 for the others.  This returns the range count that fills the
 * device once: num_cus / ceil(q_len * H / 128), at least 1. */
int mla_plan_paged(int num_cus, int B, int q_len, int H, int* num_splits);

/* Bytes of workspace mla_paged_decode needs: (num_splits + B - 1) partial slots of
 * q_len * H rows of (512 + 1) fp32 values (TokenSpeed page, module note on the decode
 * workspace: D + 1 accumulator values per split), plus 2 * B int32 split descriptors
 * and a 256-byte info block, each section rounded up to 256 bytes.  Returns 0 for
 * invalid arguments.  The workspace needs no initialisation. */
size_t mla_paged_workspace_bytes(int B, int q_len, int H, int num_splits);

/* Contiguous split-KV decode, per-split outputs (TileGym page, forward and
 * _launch_mla_decode_kernel).
 *   q        [B, H, 512] bf16     qpe [B, H, 64] bf16
 *   kv       [B, S_kv, 512] bf16  kpe [B, S_kv, 64] bf16
 *   o_part   [B, H, NS, 512] fp32 (out)  normalised partial O_j of split j
 *   lse_part [B, H, NS] fp32 (out)       lse_j (natural log; -inf for no token)
 * with NS = ceil(S_kv / kv_len_per_split); split j covers tokens
 * [j*L, min((j+1)*L, S_kv)).  kv_len_per_split must be a power of two >= 128 (the
 * page's assertions); sm_scale finite and >= 0.  H: multiple of 16, <= 128.  1 <= B <= 65535; NS <= 65535;
 * NS * B <= 2^30 (one workgroup per request and split). */
int mla_decode_splitkv(const uint16_t* q, const uint16_t* qpe, const uint16_t* kv,
                       const uint16_t* kpe, int B, int H, int S_kv, float sm_scale,
                       int kv_len_per_split, float* o_part, float* lse_part, void* stream);

/* Split-K log-sum-exp reduce (TileGym page, forward: splitk_reduce).
 *   o_part [rows, num_splits, 512] fp32, lse_part [rows, num_splits] fp32 (in)
 *   o      [rows, 512] bf16 (out, round-to-nearest-even)
 *   lse    [rows] fp32 (out; may be NULL)
 * Splits with lse_j = -inf contribute nothing, whatever their o_part holds (NaN
 * included; the buffer is still read, so it must span all rows x num_splits).  rows >= 1,
 * 1 <= num_splits <= 65536. */
int mla_splitkv_combine(const float* o_part, const float* lse_part, int rows, int num_splits,
                        uint16_t* o, float* lse, void* stream);

/* First launch of the paged decode alone: writes the split partials of every request
 * into `workspace` (same arguments and checks as mla_paged_decode, without the
 * outputs).  Range w of the num_splits ranges of the batch's tiles (64 tokens for the FP8
 * formats, 32 for the others) writes, for each request b it touches, the normalised partial O and its lse into
 * slot w + b of the workspace; the workspace also records, per request, the first and
 * last range that touch it.  Useful to a caller that merges partials itself, or times
 * the two launches apart.  Workspace layout (each section starting on a 256-byte
 * boundary, slots = num_splits + B - 1, rows = q_len * H): o_part [slots][rows][512] fp32
 * (normalised O_j), lse_part [slots][rows] fp32, seg_first [B] int32, seg_last [B]
 * int32, then an info block whose first int32 is the batch's total cost.  Only the slots
 * of ranges that hold tiles of the request are written. */
int mla_paged_decode_partials(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                              float kv_scale, int num_pages, int page_size,
                              int64_t page_stride_bytes, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* seq_lens, int B, int q_len,
                              int H, float sm_scale, int num_splits, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Second launch of the paged decode alone: merges the partials a preceding
 * mla_paged_decode_partials call on the same stream wrote into `workspace`, with the
 * same seq_lens, B, q_len, H, num_splits, max_blocks_per_seq and page_size, into
 * o [B, q_len, H, 512] bf16 and lse [B, q_len, H] fp32 (may be NULL). */
int mla_paged_combine(const void* workspace, size_t workspace_bytes, const int32_t* seq_lens, int B,
                      int q_len, int H, int num_splits, int max_blocks_per_seq, int page_size,
                      uint16_t* o, float* lse, void* stream);

/* Paged decode with split-KV and the LSE reduce, in two launches on `stream`
 * (TokenSpeed page, forward_decode / tokenspeed_mla_decode; metrale page,
 * mla_paged_decode_fp8 / mla_paged_decode_nvfp4).
 *   q            [B, q_len, H, 512] bf16    qpe [B, q_len, H, 64] bf16
 *   kv_cache     num_pages pages of page_stride_bytes each, in format `fmt`
 *   kv_scale     FP8 dequant scale (finite, > 0); ignored for other formats
 *   block_tables [B, max_blocks_per_seq] int32: token t of request b is row t % page_size
 *                of page block_tables[b, t / page_size]
 *   seq_lens     [B] int32, device: tokens of request b, counting its q_len new ones
 *   o            [B, q_len, H, 512] bf16 (out)   lse [B, q_len, H] fp32 (out; may be NULL)
 * Query i of request b sits at position seq_lens[b] - q_len + i and sees tokens
 * 0 .. seq_lens[b] - q_len + i (causal across the q_len draft tokens; all tokens when
 * q_len = 1).  Device-side preconditions: 0 <= seq_lens[b] <= max_blocks_per_seq *
 * page_size and 0 <= block_tables[b, i] < num_pages for i < ceil(seq_lens[b] /
 * page_size); entries past that are never read.  Out-of-range lengths and page indices
 * are clamped on the device, so a violation gives wrong numbers, never an access outside
 * the cache or the table.  Constraints checked on the host: fmt valid; page_size 32 or
 * 64; page_stride_bytes a multiple of 16 and at least page_size * (1152, 576 or 324)
 * bytes; sm_scale finite and >= 0; 1 <= q_len <= 8; H a multiple of 16, <= 128; 1 <= B <= 4096;
 * 1 <= num_splits <= 65536; B * max_blocks_per_seq * page_size < 2^31;
 * workspace_bytes >= mla_paged_workspace_bytes(B, q_len, H, num_splits). */
int mla_paged_decode(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                     float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                     int num_splits, void* workspace, size_t workspace_bytes, uint16_t* o,
                     float* lse, void* stream);

/* mla_paged_decode with a sliding window and per-head attention sinks (metrale page,
 * mla_paged_decode_fp8: sliding_window and sinks arguments, sinks "per-head, FP32, may be
 * null").  The page names them without defining them; this library reads them as:
 *   sliding_window  W >= 0.  W > 0: query i of request b (position seq_lens[b] - q_len + i)
 *                   sees only tokens max(0, position - W + 1) .. position.  0: no window
 *                   (the same result as mla_paged_decode).
 *   sinks           [H] fp32, device, or NULL.  sinks[h] is one more logit of head h, in the
 *                   units of the scaled scores, that joins the softmax denominator and has
 *                   no value: LSE = ln(exp(sinks[h]) + sum_t exp(s_t)),
 *                   O = sum_t exp(s_t - LSE) * latent_t.  A row that sees no token gets O = 0
 *                   and LSE = sinks[h].
 * Every other argument, and every check, is that of mla_paged_decode; in addition
 * sliding_window < 0 or a misaligned sinks pointer returns MLA_ERR_INVALID_ARG. */
int mla_paged_decode_ext(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                         float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                         int sliding_window, const float* sinks, int num_splits, void* workspace,
                         size_t workspace_bytes, uint16_t* o, float* lse, void* stream);

/* mla_paged_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments,
 * checks and results, without workspace arguments.  The workspace is a 256-byte aligned
 * array of MLA_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per GPU,
 * held from the first call on that GPU until the process ends; its device address is
 * looked up once per GPU (the GPU of `stream`, or the current one for a null stream).
 * The call allocates nothing.  The problem's workspace, mla_paged_workspace_bytes(B,
 * q_len, H, num_splits), must fit: otherwise it returns MLA_ERR_SCRATCH_LIMIT (for
 * B = 64, q_len = 1, H = 128 and 256 splits it is 84 MB; for B = 128, q_len = 2, H = 128
 * and 128 splits, 134 MB).  Every call on one GPU shares that GPU's array, and the array
 * keeps the last call's contents, which the next call does not need: calls that overlap
 * on one GPU (on different streams, or from different threads) race and must not be
 * issued. */
int mla_paged_decode_noalloc(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                             float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                             int num_splits, uint16_t* o, float* lse, void* stream);

/* Paged split planner in the pages' own split form (TileGym page,
 * _mla_decoding_split_kv.forward, with the batch's longest sequence as S_kv): from a host
 * copy of seq_lens,
 *   max_len = max(1, max_b seq_lens_host[b]);  estimate = max(1, num_cus / B);
 *   kv_len_per_split = max(next_power_of_2(max_len / estimate), 128);
 *   max_splits = ceil(max_len / kv_len_per_split).
 * kv_len_per_split is a power of two >= 128, so a multiple of either page size.  q_len and
 * page_size are checked (1..8; 32 or 64) and do not enter the formula.  Host-only integer
 * work.  Returns MLA_ERR_INVALID_ARG for max_splits > 65535. */
int mla_plan_paged_splits(int num_cus, int B, int q_len, const int32_t* seq_lens_host, int page_size,
                          int* kv_len_per_split, int* max_splits);

/* Bytes of workspace mla_paged_decode_splits needs: B * q_len * H * max_splits partials of
 * 512 + 1 fp32 values (TokenSpeed page, module note on the decode workspace: (D + 1)
 * accumulator values per split and head), laid out as o_part [B, q_len, H, max_splits, 512]
 * fp32 followed, at the next 256-byte boundary, by lse_part [B, q_len, H, max_splits] fp32.
 * Returns 0 for invalid arguments. */
size_t mla_paged_splits_workspace_bytes(int B, int q_len, int H, int max_splits);

/* Paged decode with fixed-length splits, the pages' own split form (TileGym page,
 * forward: kv_len_per_split; TokenSpeed page, forward_decode), in two launches on
 * `stream`: split j of request b covers tokens [j*L, min((j+1)*L, seq_lens[b])) of it,
 * L = kv_len_per_split, and writes its normalised partial O_j and lse_j into the workspace
 * (layout of mla_paged_splits_workspace_bytes; a split past the request's end writes only
 * lse_j = -inf); the split-K reduce then merges each row's max_splits partials into o and
 * lse.  Every other argument, precondition and result is that of mla_paged_decode (no
 * sliding window, no sinks).  Checked on the host besides mla_paged_decode's checks:
 * kv_len_per_split a power of two >= 128 (the page's assertions); 1 <= max_splits <=
 * 65535; max_splits * kv_len_per_split >= max_blocks_per_seq * page_size (the splits cover
 * every admissible length); workspace_bytes >= mla_paged_splits_workspace_bytes(B, q_len,
 * H, max_splits).  mla_plan_paged / mla_paged_decode cut the batch into cost-balanced
 * ranges instead, which keeps every workgroup busy when lengths differ. */
int mla_paged_decode_splits(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                            float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* seq_lens, int B, int q_len, int H, float sm_scale,
                            int kv_len_per_split, int max_splits, void* workspace, size_t workspace_bytes,
                            uint16_t* o, float* lse, void* stream);

/* KV-cache append: store T new tokens into the paged pool before decoding them
 * (TokenSpeed page, forward_decode: each new token's latent and rope key are written into
 * the paged pool at its cache location before attention; metrale page,
 * mla_cache_assemble: a cache row is the latent followed by the rope key).
 *   latent   [T, 512] bf16   rope [T, 64] bf16
 *   slots    [T] int32, device: token j goes to row slots[j] % page_size of page
 *            slots[j] / page_size; slots outside [0, num_pages * page_size) are skipped
 *            (padding).  Slots must be distinct.
 *   kv_cache the page pool (num_pages pages of page_stride_bytes), same layout as
 *            mla_paged_decode reads; only the addressed rows (and, for NVFP4, their scale
 *            bytes) are written.
 * Encoding: bf16 stores the bit patterns; FP8 (and MLA_KV_FP8_E4M3_QFP8, whose pages are
 * the same) stores the E4M3 code of x / kv_scale
 * (binary32 division), saturated at +-448, nearest value, ties to the even code; NVFP4
 * stores per 16 values the E4M3 code of amax / 6 as the scale and the E2M1 codes of
 * x / scale (saturated at +-6, nearest, ties to even; all zero when the scale decodes to
 * 0).  Every code keeps the sign of its scaled value.  Inputs must be finite.
 * Constraints checked on the host: T >= 0 (0 enqueues nothing); fmt valid; page_size 32
 * or 64; num_pages >= 1 and num_pages * page_size < 2^31; page_stride_bytes a multiple of
 * 16 and at least page_size * (1152, 576 or 324); kv_scale finite and > 0 for FP8;
 * latent, rope and kv_cache 16-byte aligned, slots 4-byte aligned. */
int mla_kv_append(const uint16_t* latent, const uint16_t* rope, const int32_t* slots, int T, void* kv_cache,
                  int fmt, float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
