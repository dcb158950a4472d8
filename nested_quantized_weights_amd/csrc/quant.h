// Internal: the nested quantization rule of nestspec.h (base code, then the
// residual at s/16) with its quotients formed by a reciprocal multiply,
// bit-identical to the IEEE-division rule. Shared by the KV append and the
// attention kernels that rebuild an open block from its fp32 values.
#pragma once

#include "common.h"

namespace nest {

// Round to the nearest integer of x / s by x * r (r = 1/s), taking the IEEE
// quotient only when x * r is within 1e-5 of a half-integer. For |x/s| <= 8
// both x * r and fl(x/s) are within 1e-6 of x/s, so away from a tie all
// three round alike.
__device__ __forceinline__ float rint_div(float x, float s, float r) {
  const float t = x * r;
  return (fabsf(t - floorf(t) - 0.5f) > 1.0e-5f && r < INFINITY) ? rintf(t) : rintf(x / s);
}

// nest_codes with the two quotients formed by rint_div; |w/s| <= 7 and
// |e/s16| <= 8 + 2^-20 hold by construction of s, so the codes are those of
// nest_codes bit for bit.
__device__ __forceinline__ void nest_codes_fast(float w, float s, float s16, float rs, float rs16, int& qb,
                                                int& qr) {
  if (s == 0.0f) {
    qb = 0;
    qr = 0;
    return;
  }
  int b = static_cast<int>(rint_div(w, s, rs));
  b = b < -7 ? -7 : (b > 7 ? 7 : b);
  const float e = fmaf(-s, static_cast<float>(b), w);
  int r = 0;
  if (s16 != 0.0f) {
    float u = rint_div(e, s16, rs16);
    u = u < -8.0f ? -8.0f : (u > 7.0f ? 7.0f : u);
    r = static_cast<int>(u);
  }
  qb = b;
  qr = r;
}

}  // namespace nest
