// Pieces shared by the decode kernels: LDS layout of the vector-ALU path,
// the block-wide online softmax, the fp16-window pass and the partial write.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kBlockTok = 128;   // tokens per processing block
constexpr float kNegInf = -__builtin_inff();

struct SoftmaxState {
  float m[kMaxGqa];
  float l[kMaxGqa];
};

template <int GQA>
struct Lds {
  float q[GQA][kD];                      // query * sm * log2(e)
  float ks[kBlockTok / 32][kD];          // key scale / min per (group in block, channel)
  float km[kBlockTok / 32][kD];
  int kb[kBlockTok / 32][kD];            // Kitty boosted row per (group in block, channel)
  float vs[kBlockTok * 4];               // value scale / min per (token, channel group)
  float vm[kBlockTok * 4];
  float part[2][GQA][kBlockTok];         // q.k partial sums of the two channel halves
  float p[GQA][kBlockTok];               // logits, then probabilities
  float m[GQA], l[GQA], alpha[GQA];
  float acc[GQA][kD];                    // final combine of the two token halves
  int64_t gblk[kBlockTok / 32];          // cache block (page) of each group in the block
  int bad;                               // a group's page lies outside the pool
};

// ------------------------------------------------------------------ softmax
// Block-wide online softmax update over the nt logits in lds.p.
template <int GQA>
__device__ void softmax_block(Lds<GQA>& s, int nt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < GQA; h += kThreads / 64) {
    float mx = kNegInf;
    for (int t = lane; t < nt; t += 64) mx = fmaxf(mx, s.p[h][t]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_old = s.m[h];
    const float m_new = fmaxf(m_old, mx);
    float sum = 0.f;
    for (int t = lane; t < nt; t += 64) {
      const float e = exp2f(s.p[h][t] - m_new);
      s.p[h][t] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      const float alpha = exp2f(m_old - m_new);   // 0 when m_old == -inf
      s.alpha[h] = alpha;
      s.l[h] = s.l[h] * alpha + sum;
      s.m[h] = m_new;
    }
  }
}

// ------------------------------------------------------------ fp16 window
// Window tokens [u0, u0+nt) of the concatenation sink | residual.
template <int GQA>
__device__ void window_block(const DecodeArgs& a, Lds<GQA>& s, int64_t head, int u0, int nt,
                             float (&acc)[GQA]) {
  const int tid = threadIdx.x;
  auto krow = [&](int u) -> const uint16_t* {
    return u < a.n_sink ? a.k_sink + (head * a.sink_cap + u) * kD
                        : a.k_res + (head * a.res_cap + (u - a.n_sink)) * kD;
  };
  auto vrow = [&](int u) -> const uint16_t* {
    return u < a.n_sink ? a.v_sink + (head * a.sink_cap + u) * kD
                        : a.v_res + (head * a.res_cap + (u - a.n_sink)) * kD;
  };
  {
    const int t = tid & (kBlockTok - 1), half = tid >> 7;
    if (t < nt) {
      const uint16_t* k = krow(u0 + t) + half * (kD / 2);
      float dot[GQA];
#pragma unroll
      for (int h = 0; h < GQA; ++h) dot[h] = 0.f;
      for (int c = 0; c < kD / 2; ++c) {
        const float x = h2f(k[c]);
#pragma unroll
        for (int h = 0; h < GQA; ++h) dot[h] = fmaf(s.q[h][half * (kD / 2) + c], x, dot[h]);
      }
#pragma unroll
      for (int h = 0; h < GQA; ++h) s.part[half][h][t] = dot[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < GQA * nt; i += kThreads) {
    const int h = i / nt, t = i % nt;
    s.p[h][t] = s.part[0][h][t] + s.part[1][h][t];
  }
  __syncthreads();
  softmax_block<GQA>(s, nt);
  __syncthreads();
  {
    const int d = tid & (kD - 1), half = tid >> 7;
#pragma unroll
    for (int h = 0; h < GQA; ++h) acc[h] *= s.alpha[h];
    const int tb = half * (kBlockTok / 2);
    const int te = min(nt, tb + kBlockTok / 2);
    for (int t = tb; t < te; ++t) {
      const float x = h2f(vrow(u0 + t)[d]);
#pragma unroll
      for (int h = 0; h < GQA; ++h) acc[h] = fmaf(s.p[h][t], x, acc[h]);
    }
  }
  __syncthreads();
}

// Combine the two token halves of the accumulators and write (m, l, acc) of
// part `part` for every query head of kv head hk.
template <int GQA>
__device__ void write_partial(const DecodeArgs& a, Lds<GQA>& s, int64_t b, int64_t hk, int part,
                              const float (&acc)[GQA]) {
  const int tid = threadIdx.x;
  const int d = tid & (kD - 1), half = tid >> 7;
  const int n_parts = a.n_parts;
  if (half) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) s.acc[h][d] = acc[h];
  }
  __syncthreads();
  if (tid == 0 && s.bad) status_add(a.status, kStatusBadPage);
  if (!half) {
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      float* w = a.ws + (((b * a.H_q) + hk * GQA + h) * n_parts + part) * (kD + 2);
      // a bad page poisons the part: l = 1 keeps it in the merge, acc NaN
      w[2 + d] = s.bad ? __builtin_nanf("") : acc[h] + s.acc[h][d];
      if (d == 0) {
        w[0] = s.bad ? 0.f : s.m[h];
        w[1] = s.bad ? 1.f : s.l[h];
      }
    }
  }
}

}  // namespace
}  // namespace kvq
