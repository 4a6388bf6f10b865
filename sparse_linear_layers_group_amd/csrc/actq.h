// actq.h -- device helpers of the per-token int8 activation quantiser,
// shared by the activation kernels and the fused decode prologue so that
// both give bit-identical codes.
#pragma once

#include "common.h"

namespace bl {

// x_q = rint(127 x / a) with a correctly rounded binary32 division: 127 x
// is exact in binary32, and a quotient of two 8-bit-significand values that
// is not a half-integer sits at least ~2^-16 (relative) away from one, far
// beyond binary32 rounding, so rint (ties to even) of the rounded quotient
// equals round-half-even of the exact quotient.  |x_q| <= 127, so the clip
// to [-128, 127] never binds.  a = 0 gives zero codes.
__device__ __forceinline__ uint2 quant8(const uint4& v, float a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t q[2] = {0, 0};
  if (a > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
      const int qi = (int)rintf((127.0f * x) / a);
      q[j >> 2] |= ((uint32_t)qi & 0xffu) << (8 * (j & 3));
    }
  }
  return make_uint2(q[0], q[1]);
}

// max |x| over 8 bf16 values
__device__ __forceinline__ float absmax8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  return a;
}

}  // namespace bl
