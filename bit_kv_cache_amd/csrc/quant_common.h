// Device helpers of the min-max group quantizer shared by the quantize kernel
// and the decode kernel's fused append (not installed).
#pragma once

#include "kvq_internal.h"

namespace kvq {

// Code of x in a group with min mn and stored scale s (rs within one ulp of
// 1/s: the IEEE reciprocal, or v_rcp_f32): round-half-even(clamp((x - mn)/s,
// 0, maxq)) with the IEEE fp32 quotient (KIVI page, Step 1).  The quotient
// is taken as (x - mn) * rs, falling back to the IEEE division near a
// rounding tie.  Exact: the range fits (x - mn)/s <= 1.5 maxq (s is the
// fp16-rounded range/maxq, at least 2^-24 when nonzero).  The product is
// within a relative 1.5 * 2^-23 of the true quotient (2^-23 from rs, 2^-24
// from its own rounding) and the IEEE quotient within half an ulp of it, so
// the two differ by less than 2^-17 for maxq <= 15 (quotients <= 22.5) and
// less than 2^-13 for maxq = 255 (quotients <= 383); round-half-even of two
// values that close differs only when a half-integer lies between them, so
// the fallback window is 2^-16 for 2- and 4-bit codes and 2^-12 for 8-bit
// ones.  The clamp bounds are integers and cannot change that.  s == 0 (max
// == min, or a range whose scale underflows fp16) gives code 0.
__device__ __forceinline__ uint32_t quant_code_rcp(float x, float mn, float s, float rs,
                                                   float maxq) {
#pragma clang fp contract(off)
  if (s == 0.0f) return 0u;
  const float dlt = x - mn;
  float y = dlt * rs;
  const float win = maxq > 15.0f ? 0x1p-12f : 0x1p-16f;
  if (__builtin_fabsf((y - __builtin_floorf(y)) - 0.5f) < win) y = dlt / s;
  y = fminf(fmaxf(y, 0.0f), maxq);
  return (uint32_t)__builtin_rintf(y);
}

// Exact code by the IEEE quotient (the reference form of quant_code_rcp).
__device__ __forceinline__ uint32_t quant_code_div(float x, float mn, float s, float maxq) {
#pragma clang fp contract(off)
  if (s == 0.0f) return 0u;
  float y = (x - mn) / s;
  y = fminf(fmaxf(y, 0.0f), maxq);
  return (uint32_t)__builtin_rintf(y);
}

// fp16 scale of a group from its min and max: fp16((max - min)/maxq), the
// subtraction and division in IEEE fp32, both rounded to nearest even.
__device__ __forceinline__ uint16_t group_scale(float mn, float mx, float maxq) {
#pragma clang fp contract(off)
  return f2h((mx - mn) / maxq);
}

}  // namespace kvq
