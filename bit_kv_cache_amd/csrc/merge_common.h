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
  if constexpr (NPM <= 8) {
#pragma unroll
    for (int j = 0; j < NPM; ++j) {
      const float* wp = w + (int64_t)min(j, np - 1) * (kD + 2);
      m[j] = ld(wp);
      l[j] = ld(wp + 1);
      v[j] = ld(wp + 2 + d);
    }
  } else {
    // the same loads with a per-lane pointer stepped part by part (many
    // parts' wave-uniform offsets would otherwise crowd the scalar registers)
    const float* wp = w;
#pragma unroll
    for (int j = 0; j < NPM; ++j) {
      m[j] = ld(wp);
      l[j] = ld(wp + 1);
      v[j] = ld(wp + 2 + d);
      wp += j + 1 < np ? kD + 2 : 0;
    }
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

// A block's record (m, l, acc[d]) of part `part` of row bh, stored for the
// in-launch merge (device-scope stores, read by another block of the launch)
// or for a merge launch (plain stores).
__device__ __forceinline__ void store_record(const DecodeArgs& a, int64_t bh, int part, int d,
                                             float m, float l, float v) {
  float* wp = a.ws + (bh * a.n_parts + part) * (kD + 2);
  if (a.counters) {
    __hip_atomic_store(wp + 2 + d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(wp, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(wp + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    wp[2 + d] = v;
    if (d == 0) {
      wp[0] = m;
      wp[1] = l;
    }
  }
}

// In-launch merge (decode kernels with one part per block, at most 32 parts):
// after a block has stored its records with store_record, its arrival on the
// head's counter, and in the last block of the head to arrive, the
// log-sum-exp merge of the head's GQA query rows into the output.  No block
// waits for another, so the order in which blocks run is free.  The last
// block resets the counter, leaving it zero for the next call.  last_flag is
// an LDS word of the block.
template <int GQA, int MAXP = kFusedMergeParts>
__device__ __forceinline__ void merge_in_launch(const DecodeArgs& a, int64_t b, int64_t hk,
                                                int head32, int& last_flag) {
  // this thread's stores have completed (they are visible device-wide)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + head32, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == a.n_parts - 1;   // a head's blocks, one part each
    if (last) __hip_atomic_store(a.counters + head32, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = last;
  }
  __syncthreads();
  if (!last_flag) return;
  const int np = a.n_parts;
  for (int i = threadIdx.x; i < GQA * kD; i += blockDim.x) {
    const int64_t bh = b * a.H_q + hk * GQA + i / kD;
    const int d = i % kD;
    if constexpr (MAXP <= 8) {
      if (np <= 4) merge_row<4, true>(a.ws, np, a.out, bh, d);
      else merge_row<8, true>(a.ws, np, a.out, bh, d);
    } else {
      static_assert(MAXP == kPwFusedMergeParts, "up to 32 parts");
      if (np <= 16) merge_row<16, true>(a.ws, np, a.out, bh, d);
      else merge_row<32, true>(a.ws, np, a.out, bh, d);
    }
  }
}

}  // namespace kvq
