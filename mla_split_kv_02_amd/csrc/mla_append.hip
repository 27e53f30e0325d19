// KV-cache append for gfx950: store each new token's 576-wide row [latent | rope] into
// its slot of the paged pool, in the pool's format.  This is the write that precedes the
// decode (TokenSpeed page, forward_decode: the new tokens' latent and rope key go into
// the paged pool at their cache locations before attention; metrale page,
// mla_cache_assemble: one token's row is the latent followed by the rope key).
//
// Encoding (the same readings as the FP8 / NVFP4 page layouts the decode reads):
//   bf16   the bit patterns, unchanged;
//   FP8    E4M3 "FN" code of y = x / kv_scale (binary32 division), saturated at +-448,
//          nearest value with ties to the even code;
//   NVFP4  per 16 values: scale code = E4M3 code of amax / 6 (as above), scale value s
//          its decoded value; data = E2M1 code of x / s, saturated at +-6, nearest value
//          with ties to the even code; all data codes 0 when s is 0.
// The sign of the scaled value is kept in every code (a negative value that rounds to
// zero stores negative zero).  Inputs must be finite.
//
// One wavefront per token; lane g < 36 owns values 16g .. 16g+15 (latent for g < 32,
// rope after), which is also one NVFP4 scale group, so no lane exchanges data.

#include "mla_fp8.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int kGroups = kRow / 16;  // 36 groups of 16 values per row

// E2M1 code of a finite binary32 value: the magnitude thresholds between the values
// 0, .5, 1, 1.5, 2, 3, 4, 6 (a midpoint goes to the even code: > on the way to an odd
// code, >= on the way to an even one); above 5 it saturates at 6.
__device__ __forceinline__ unsigned e2m1_code(float y) {
  const float a = fabsf(y);
  const unsigned mag = (unsigned)(a > 0.25f) + (unsigned)(a >= 0.75f) + (unsigned)(a > 1.25f) +
                       (unsigned)(a >= 1.75f) + (unsigned)(a > 2.5f) + (unsigned)(a >= 3.5f) +
                       (unsigned)(a > 5.0f);
  return ((__float_as_uint(y) >> 28) & 0x8u) | mag;
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void kv_append_kernel(const AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= p.T || lane >= kGroups) return;
  const int slot = p.slots[j];
  if (slot < 0 || (int64_t)slot >= (int64_t)p.num_pages * p.page_size) return;
  const int page = slot / p.page_size, row = slot - page * p.page_size;
  uint8_t* const base = p.cache + (int64_t)page * p.page_stride;

  // values 16 lane .. 16 lane + 15 as 8 bf16 pairs
  const uint16_t* src = lane < 32 ? p.latent + (int64_t)j * kLatent + 16 * lane
                                  : p.rope + (int64_t)j * kRope + 16 * (lane - 32);
  const u32x4 w0 = reinterpret_cast<const u32x4*>(src)[0];
  const u32x4 w1 = reinterpret_cast<const u32x4*>(src)[1];
  const unsigned w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};

  if (p.fmt == kFmtBf16) {
    u32x4* dst = reinterpret_cast<u32x4*>(base + (int64_t)row * (2 * kRow) + 32 * lane);
    dst[0] = w0;
    dst[1] = w1;
  } else if (p.fmt == kFmtFp8) {
    unsigned out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned c0 = e4m3_code(__fdiv_rn(bf16_lo(w[i]), p.kv_scale));
      const unsigned c1 = e4m3_code(__fdiv_rn(bf16_hi(w[i]), p.kv_scale));
      out[i >> 1] |= (c0 | (c1 << 8)) << (16 * (i & 1));
    }
    *reinterpret_cast<u32x4*>(base + (int64_t)row * kRow + 16 * lane) = u32x4{out[0], out[1], out[2], out[3]};
  } else {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
    const unsigned sc = e4m3_code(__fdiv_rn(amax, 6.0f));
    const float s = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc, false)[0];  // exact decode
    unsigned out[2] = {0, 0};
    if (s > 0.f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned c0 = e2m1_code(__fdiv_rn(bf16_lo(w[i]), s));
        const unsigned c1 = e2m1_code(__fdiv_rn(bf16_hi(w[i]), s));
        out[i >> 2] |= (c0 | (c1 << 4)) << (8 * (i & 3));  // even value in the low nibble
      }
    }
    *reinterpret_cast<u32x2*>(base + (int64_t)row * (kRow / 2) + 8 * lane) = u32x2{out[0], out[1]};
    base[(int64_t)p.page_size * (kRow / 2) + (int64_t)row * kGroups + lane] = (uint8_t)sc;
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
