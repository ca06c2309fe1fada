// Log-sum-exp merge of split-K partials, one (batch, query head) row, shared
// by the merge kernel and the merge + append kernel (not installed).
#pragma once

#include "kvq_internal.h"

namespace kvq {

// Row bh of the partials [rows][n_parts][D+2] (m, l, acc[D]) into out[bh][d]
// for the calling thread's channel d: M = max of m_p over the parts with
// l_p > 0, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p (0 when every
// part is empty).  Up to NPM parts; every load is issued up front (indices
// past the count re-read the last part and get weight 0), so the merge costs
// one memory round trip.
//
// COHERENT: the partials were written by other blocks of the same launch
// (possibly on other XCDs, whose L2 caches are not coherent with this one):
// read them with device-scope relaxed atomic loads, which the writers paired
// with device-scope stores.
template <int NPM, bool COHERENT = false>
__device__ __forceinline__ void merge_row(const float* ws, int np, float* out, int64_t bh, int d) {
  const float* w = ws + bh * (int64_t)np * (kD + 2);
  auto ld = [](const float* p) -> float {
    if constexpr (COHERENT)
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      return *p;
  };
  float m[NPM], l[NPM], v[NPM];
#pragma unroll
  for (int j = 0; j < NPM; ++j) {
    const float* wp = w + (int64_t)min(j, np - 1) * (kD + 2);
    m[j] = ld(wp);
    l[j] = ld(wp + 1);
    v[j] = ld(wp + 2 + d);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < NPM; ++j)
    if (j < np && l[j] > 0.f) M = fmaxf(M, m[j]);
  // weights select rather than branch, so the loads stay unconditional (an
  // excluded part's values are finite: empty parts hold zeros)
  float L = 0.f, o = 0.f;
#pragma unroll
  for (int j = 0; j < NPM; ++j) {
    const float f = (j < np && l[j] > 0.f) ? exp2f(m[j] - M) : 0.f;
    L = fmaf(l[j], f, L);
    o = fmaf(v[j], f, o);
  }
  out[bh * kD + d] = L > 0.f ? o / L : 0.f;
}

}  // namespace kvq
