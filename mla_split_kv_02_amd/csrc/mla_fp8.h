// E4M3 ("FN") encoding on the device, shared by the cache append and the FP8-query
// decode.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

namespace mla {

// E4M3 code of a finite binary32 value: saturate at 448, round the magnitude to 3
// mantissa bits (nearest, ties to even) on the binary32 bits for normal results
// (>= 2^-6), on the 2^-9 subnormal grid below; the carry out of the mantissa moves into
// the exponent, which is rebased from 127 to 7.  The sign of y is kept.  Both roundings
// are computed and one is selected, so the code has no branch.
__device__ __forceinline__ unsigned e4m3_code(float y) {
  const unsigned sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  const unsigned u = __float_as_uint(a);
  const unsigned normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  const unsigned subnormal = (unsigned)__builtin_rintf(a * 512.0f);  // 0 .. 8 (8 is 2^-6)
  return sign | (a < 0.015625f ? subnormal : normal);
}

}  // namespace mla
