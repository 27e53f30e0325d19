// mla_paged_decode_noalloc: the paged decode with its workspace in a file-scope device
// array instead of caller memory, for callers that cannot allocate.  Every GPU that runs
// this library holds its own copy of the array until the process ends; the host finds
// that copy's address once per device (hipGetSymbolAddress, with the device current) and
// hands it to the ordinary paged decode as its workspace.  The array's host-side name is
// never used as a device address.

#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;

// The workspace of mla_paged_decode: partial slots, split descriptors and the info block.
// It needs no initialisation (the decode launch writes everything the combine reads), so
// whatever an earlier call left in it does not matter.
__device__ __attribute__((aligned(256))) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device).
int scratch_of(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[device]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MLA_ERR_HIP;
    if (cur != device && hipSetDevice(device) != hipSuccess) return MLA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return MLA_ERR_HIP;
    g_scratch[device] = ptr;
  }
  *out = g_scratch[device];
  return MLA_OK;
}

}  // namespace

extern "C" int mla_paged_decode_noalloc(const uint16_t* q, const uint16_t* qpe, const void* kv_cache, int fmt,
                                        float kv_scale, int num_pages, int page_size, int64_t page_stride_bytes,
                                        const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                                        int B, int q_len, int H, float sm_scale, int num_splits, uint16_t* o,
                                        float* lse, void* stream) {
  if (!q || !qpe || !kv_cache || !block_tables || !seq_lens || !o) return MLA_ERR_INVALID_ARG;
  const size_t need = mla_paged_workspace_bytes(B, q_len, H, num_splits);
  if (need == 0) return MLA_ERR_INVALID_ARG;
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH_LIMIT;
  // the device the work runs on: the stream's, or the current one for the null stream
  int device = -1;
  if (stream) {
    if (hipStreamGetDevice((hipStream_t)stream, &device) != hipSuccess) return MLA_ERR_HIP;
  } else if (hipGetDevice(&device) != hipSuccess) {
    return MLA_ERR_HIP;
  }
  void* ws = nullptr;
  const int st = scratch_of(device, &ws);
  if (st != MLA_OK) return st;
  return mla_paged_decode(q, qpe, kv_cache, fmt, kv_scale, num_pages, page_size, page_stride_bytes, block_tables,
                          max_blocks_per_seq, seq_lens, B, q_len, H, sm_scale, num_splits, ws,
                          (size_t)MLA_NOALLOC_SCRATCH_BYTES, o, lse, stream);
}
