// Measured ceilings of the MI355X for the benchmark's roofline fractions: a stream-read
// kernel (the HBM bandwidth a plain coalesced read reaches) and MFMA loops (the matrix-core
// rate a kernel doing nothing else reaches, bf16 and f16 32x32x16, FP8 32x32x64).  Built into
// libmla_ceiling.so, apart from the decode library; nothing in the decode path calls it.

#include "mla_ceiling.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kReadThreads = 256;
constexpr int kUnroll = 8;

// Thread g reads the 16-byte chunks g, g + G, g + 2G, .. (G = grid threads), kUnroll loads
// in flight, and writes the XOR of everything it read to out[g].
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* buf, int64_t n16, uint32_t* out) {
  const int64_t g = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  const int64_t G = (int64_t)gridDim.x * kReadThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = g;
  for (; i + (kUnroll - 1) * G < n16; i += kUnroll * G) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * G);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += G) acc ^= buf[i];
  out[g] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Each wavefront runs `iters` rounds of four independent MFMA chains and writes one sum.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out, int seed) {
  const int lane = threadIdx.x & 63;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)((lane + e + seed) & 7));
      b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(a), "v"(b));
    }
  } else if (KIND == 2) {
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (_Float16)(0.001f * (float)((lane + e + seed) & 7));
      b[e] = (_Float16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i) {
      asm volatile(
          "v_mfma_f32_32x32x16_f16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_f16 %1, %4, %5, %1\n\t"
          "v_mfma_f32_32x32x16_f16 %2, %4, %5, %2\n\t"
          "v_mfma_f32_32x32x16_f16 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(a), "v"(b));
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x20202020 + ((lane + e + seed) & 7);
      b[e] = 0x18181818 + ((lane * 3 + e) & 7);
    }
    for (int i = 0; i < iters; ++i) {
      asm volatile(
          "v_mfma_f32_32x32x64_f8f6f4 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x64_f8f6f4 %1, %4, %5, %1\n\t"
          "v_mfma_f32_32x32x64_f8f6f4 %2, %4, %5, %2\n\t"
          "v_mfma_f32_32x32x64_f8f6f4 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(a), "v"(b));
    }
  }
  // wait states before the results are read by vector instructions
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  if (lane == 0) out[(int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int mla_ceiling_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!buf || !out || blocks < 1 || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_ceiling_mfma(int kind, int iters, float* out, int blocks, void* stream) {
  if (!out || blocks < 1 || iters < 1 ||
      (kind != MLA_CEILING_MFMA_BF16 && kind != MLA_CEILING_MFMA_FP8 && kind != MLA_CEILING_MFMA_F16))
    return -1;
  if (kind == MLA_CEILING_MFMA_BF16)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out, 1);
  else if (kind == MLA_CEILING_MFMA_F16)
    hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out, 1);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out, 1);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double mla_ceiling_mfma_flops(int kind) {
  if (kind == MLA_CEILING_MFMA_BF16 || kind == MLA_CEILING_MFMA_F16) return 2.0 * 32 * 32 * 16;
  if (kind == MLA_CEILING_MFMA_FP8) return 2.0 * 32 * 32 * 64;
  return 0.0;
}

}  // extern "C"
