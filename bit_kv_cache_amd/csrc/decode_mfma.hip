// Split-K decode attention with matrix cores (gfx950 MFMA) for GQA query
// groups of 4 or 8 heads, group size 128, head dim 128.
//
// The query heads that share a kv head form a real dense contraction with the
// kv tile (BitDecoding page, section V.A: the query group becomes the GEMM M
// dimension), so q.K^T and p.V run as v_mfma_f32_16x16x32_f16:
//
//  * B operand = packed codes, converted with one AND per two codes: a code c
//    at bit offset p (< 10) of a 16-bit half, with every other bit cleared, IS
//    the fp16 subnormal c * 2^(p-24).  Keys are packed along channels and
//    values along tokens (the contraction axes), so a lane's 32-bit word
//    holds 16 (2-bit) or 8 (4-bit) consecutive contraction indices and feeds
//    its MFMA operand with no cross-lane shuffle.  The in-word code order is
//    folded into the A operand's K-slot order.
//  * A operand = the dequantization scales folded into the query / the
//    probabilities (KIVI page Step 4: x = code*scale + min, distributed over
//    the dot product):
//        q.k_t = sum_d (q_d s_d) code_td + sum_d q_d mn_d
//        p.v_d = sum_t (p_t s_t) code_td + sum_t p_t mn_t
//    times 2^(24-p) per K slot, split into fp16 hi + lo rows (about 22
//    significant bits), with a per-group power-of-two exponent that keeps
//    every A value below 2^15.  Products are exact in the fp32 accumulator.
//  * sum_d q_d mn_d (keys) is one more MFMA per group; sum_t p_t mn_t
//    (values) is a per-head scalar kept beside the accumulator.
//
// Work split: block = 4 waves on one (batch, kv head) and one chunk of groups;
// each wave owns whole groups (round robin), keeps its own online softmax
// state, and the 4 waves are merged at the end of the chunk.  Part 0 of each
// head is the fp16 sink + residual window (vector ALU path).

#include "kvq_internal.h"
#include "decode_common.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kG = 128;          // tokens per group (the only group size built here)
constexpr int kWaves = 4;
constexpr int kThreadsM = 64 * kWaves;
constexpr float kNegInfM = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// 2-bit word (codes 0..15 at bits 2i) -> two operand quads.  Element pairs
// (lo half, hi half): j=0..7 -> codes (j, j+8) at in-half bit offset
// p(j) = {0,2,4,6,8,0,2,4}; quad q0 holds j = 0..3, quad q1 holds j = 4..7.
__device__ __forceinline__ void conv2(uint32_t w, u32x4& q0, u32x4& q1) {
  const uint32_t s = w >> 10;
  q0 = u32x4{w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
  q1 = u32x4{w & 0x03000300u, s & 0x00030003u, s & 0x000C000Cu, s & 0x00300030u};
}

// 4-bit word (codes 0..7 at bits 4i) -> one operand quad: pair r holds codes
// (r, r+4) at in-half bit offset 0 (r even) or 4 (r odd).
__device__ __forceinline__ u32x4 conv4(uint32_t w) {
  const uint32_t s = w >> 8;
  return u32x4{w & 0x000F000Fu, w & 0x00F000F0u, s & 0x000F000Fu, s & 0x00F000F0u};
}

// Contraction index (channel for keys, token-in-group for values) of element
// e (0..7) of operand chunk (c, kq): the lane group kq of K-step c.
template <int BITS>
__device__ __forceinline__ int chunk_index(int c, int kq, int e) {
  const int r = e >> 1, half = e & 1;
  if (BITS == 2) return 32 * kq + 16 * (c >> 1) + 4 * (c & 1) + r + 8 * half;
  return 32 * kq + 8 * c + r + 4 * half;
}

// Bit offset, inside its fp16 half, of the code of contraction index i.
template <int BITS>
__device__ __forceinline__ int code_offset(int i) {
  if (BITS == 2) {
    const int j = i & 7;
    return j < 5 ? 2 * j : 2 * (j - 5);
  }
  return (i & 1) ? 4 : 0;
}

__device__ __forceinline__ float exp2i(int e) {  // 2^e, e in [-126, 127]
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// smallest e with x < 2^e for x >= 0 finite (x == 0 -> -126)
__device__ __forceinline__ int ceil_exp(float x) {
  const int b = (int)((__builtin_bit_cast(uint32_t, x) >> 23) & 0xFF);
  return b == 0 ? -126 : b - 126;
}

// hi/lo fp16 split of 8 fp32 values into two operand quads (pairs e=2r,2r+1)
__device__ __forceinline__ void split_hilo(const float (&v)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(v[2 * r], v[2 * r + 1]);
    const float h0 = (float)h[0], h1 = (float)h[1];
    const auto l = __builtin_amdgcn_cvt_pkrtz(v[2 * r] - h0, v[2 * r + 1] - h1);
    hi[r] = __builtin_bit_cast(uint32_t, h);
    lo[r] = __builtin_bit_cast(uint32_t, l);
  }
}

__device__ __forceinline__ float wave_max16(float v) {  // over the 16 lanes of a row
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  return fmaxf(v, __shfl_xor(v, 8));
}

template <int GQA>
struct WaveLds {
  static constexpr int ROWS = 2 * GQA;             // A rows: (head, hi/lo)
  u32x4 ak[4][4][ROWS];                            // key A operand [c][kq][row]
  u32x4 av[4][4][ROWS];                            // value A operand [c][kq][row]
  float p[GQA][kG];                                // probabilities of the group
  float alpha[GQA];
  float m[GQA];
};

template <int GQA>
struct MergeLds {
  float num[kWaves][GQA][kD];
  float m[kWaves][GQA], l[kWaves][GQA], mt[kWaves][GQA];
};

template <int GQA>
union MfmaLds {
  struct {
    WaveLds<GQA> w[kWaves];
    u32x4 zero;
  } main;
  MergeLds<GQA> merge;
  Lds<GQA> window;
};

template <int BITS, int GQA>
__global__ __launch_bounds__(kThreadsM, 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int FPI = 32 / BITS;
  constexpr int WPT = kD / FPI;          // key words per token
  constexpr int TPC = GQA == 4 ? 2 : 1;  // tiles per QK accumulator (row slots)
  constexpr int NFRAG = 8 / TPC;         // QK accumulators per group
  constexpr int NH = GQA / 4;            // A-prep heads per lane (1 or 2)
  __shared__ MfmaLds<GQA> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;   // operand lane coordinates
  const int64_t head = blockIdx.y;
  const int64_t b = head / a.H_kv, hk = head % a.H_kv;
  const int n_parts = a.n_chunks + 1;

  // ---------------------------------------------------------------- fp16 windows
  if (blockIdx.x == 0) {
    Lds<GQA>& s = sh.window;
    for (int i = tid; i < GQA * kD; i += kThreadsM) {
      const int h = i / kD, d = i % kD;
      s.q[h][d] = h2f(a.q[((b * a.H_q) + hk * GQA + h) * kD + d]) * a.qscale;
    }
    if (tid < GQA) {
      s.m[tid] = kNegInfM;
      s.l[tid] = 0.f;
    }
    __syncthreads();
    float acc[GQA];
#pragma unroll
    for (int h = 0; h < GQA; ++h) acc[h] = 0.f;
    const int n_win = a.n_sink + a.n_res;
    for (int u = 0; u < n_win; u += kBlockTok)
      window_block<GQA>(a, s, head, u, min(kBlockTok, n_win - u), acc);
    write_partial<GQA>(a, s, b, hk, a.n_chunks, acc);
    return;
  }

  // ---------------------------------------------------------------- quantized chunk
  const int chunk = blockIdx.x - 1;
  const int64_t gb = (int64_t)chunk * a.groups_per_chunk;
  const int64_t ge = min<int64_t>(a.n_groups, gb + a.groups_per_chunk);
  WaveLds<GQA>& L = sh.main.w[wave];
  if (tid == 0) sh.main.zero = u32x4{0u, 0u, 0u, 0u};

  // query in the log2 domain, this wave's A-prep heads and chunk
  const int ph = lane >> 4;                 // A-prep head (plus 4 for the second)
  const int pc = lane & 3, pkq = (lane >> 2) & 3;   // A-prep chunk (c, kq)
  float qhat[NH][8];                        // q * sm * log2e * 2^(24 - offset)
  float qmax = 0.f;
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int h = ph + 4 * j;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = chunk_index<BITS>(pc, pkq, e);
      const float qv = h2f(a.q[((b * a.H_q) + hk * GQA + h) * kD + ch]) * a.qscale;
      qhat[j][e] = qv * exp2i(24 - code_offset<BITS>(ch));
      qmax = fmaxf(qmax, fabsf(qhat[j][e]));
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, o));
  const int e_q = ceil_exp(qmax);

  // bias operand: hi/lo of q*sm*log2e in natural channel order, rows (head, hi/lo)
  u32x4 abias[4];
  {
    const int m = lane & 15;
    const int h = (m % (2 * GQA)) >> 1, hl = m & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = h2f(a.q[((b * a.H_q) + hk * GQA + h) * kD + 32 * c + 8 * kq + e]) * a.qscale;
      u32x4 hi, lo;
      split_hilo(v, hi, lo);
      abias[c] = hl ? lo : hi;
    }
  }

  // per-wave online softmax state: this lane's QK heads hA, hB
  const int rq = lane >> 4;
  const int hA = GQA == 4 ? 2 * (rq & 1) : 2 * rq;
  float m_run[2] = {kNegInfM, kNegInfM};
  float l_part[2] = {0.f, 0.f};
  float mterm[NH];                          // sum_t p_t * value min, A-prep heads
#pragma unroll
  for (int j = 0; j < NH; ++j) mterm[j] = 0.f;
  int e_v = -1000;                          // running value-side exponent
  f32x4 acc[8];                             // p.V accumulators, 8 channel blocks
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const uint32_t* kw_base = reinterpret_cast<const uint32_t*>(a.c.k_codes);
  for (int64_t g = gb + wave; g < ge; g += kWaves) {
    // ---- loads
    const int64_t tok0 = head * a.c.t_cap + g * kG;
    uint32_t kwords[8][BITS == 2 ? 2 : 4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t* p = kw_base + (tok0 + 16 * t + n) * WPT + (BITS == 2 ? 2 : 4) * kq;
      if (BITS == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        kwords[t][0] = v[0];
        kwords[t][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < (BITS == 2 ? 2 : 4); ++i) kwords[t][i] = v[i];
      }
    }
    constexpr int VR = BITS == 2 ? 2 : 4;   // value word rows per lane group
    u32x4 vwords[VR][2];
    {
      const uint32_t* vb = reinterpret_cast<const uint32_t*>(a.c.v_codes) +
                           (head * (a.c.t_cap / FPI) + g * (kG / FPI) + VR * kq) * kD + 4 * n;
#pragma unroll
      for (int i = 0; i < VR; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          vwords[i][e] = *reinterpret_cast<const u32x4*>(vb + i * kD + 64 * e);
    }
    const int64_t kmeta = (head * (a.c.t_cap / kG) + g) * kD;
    u32x4 kmin[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kmin[c] = *reinterpret_cast<const u32x4*>(a.c.k_min + kmeta + 32 * c + 8 * kq);
    // key scales of the A-prep chunk, value scale/min of the P' chunk
    float ks[8];
    uint16_t vsb[8], vmb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = chunk_index<BITS>(pc, pkq, e);
      ks[e] = h2f(a.c.k_scale[kmeta + i]);
      vsb[e] = a.c.v_scale[head * a.c.t_cap + g * kG + i];
      vmb[e] = a.c.v_min[head * a.c.t_cap + g * kG + i];
    }

    // ---- key A operand: (q s) 2^(24-offset) 2^-E_K, hi/lo rows, via LDS
    float smax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) smax = fmaxf(smax, ks[e]);
    smax = wave_max16(smax);
    const int e_k = e_q + ceil_exp(smax) - 15;
    const float sk = exp2i(max(-126, min(127, -e_k)));
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = qhat[j][e] * ks[e] * sk;
      u32x4 hi, lo;
      split_hilo(v, hi, lo);
      const int h = ph + 4 * j;
      L.ak[pc][pkq][2 * h] = hi;
      L.ak[pc][pkq][2 * h + 1] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- bias: sum_d q_d mn_d per head (natural channel order)
    f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) cb = mfma(abias[c], kmin[c], cb);
    const float biasA = cb[0] + cb[1], biasB = cb[2] + cb[3];

    // ---- q.K^T
    const float ek = exp2i(max(-126, min(127, e_k)));
    const int m_row = lane & 15;
    float logit[NFRAG][2];
#pragma unroll
    for (int f = 0; f < NFRAG; ++f) {
      f32x4 cq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int slot = 0; slot < TPC; ++slot) {
        const int t = f * TPC + slot;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 bq;
          if (BITS == 2) {
            u32x4 q0, q1;
            conv2(kwords[t][c >> 1], q0, q1);
            bq = (c & 1) ? q1 : q0;
          } else {
            bq = conv4(kwords[t][c]);
          }
          u32x4 aq;
          if (TPC == 1) {
            aq = L.ak[c][kq][m_row];
          } else {
            const bool mine = (m_row >> 3) == slot;
            aq = mine ? L.ak[c][kq][m_row & 7] : sh.main.zero;
          }
          cq = mfma(aq, bq, cq);
        }
      }
      logit[f][0] = fmaf(cq[0] + cq[1], ek, biasA);
      logit[f][1] = fmaf(cq[2] + cq[3], ek, biasB);
    }

    // ---- online softmax over the group (per head, this wave)
    float mx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = logit[0][j];
#pragma unroll
      for (int f = 1; f < NFRAG; ++f) v = fmaxf(v, logit[f][j]);
      v = wave_max16(v);
      if (GQA == 4) v = fmaxf(v, __shfl_xor(v, 32));
      mx[j] = v;
    }
    float alpha[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float m_new = fmaxf(m_run[j], mx[j]);
      alpha[j] = exp2f(m_run[j] - m_new);
      m_run[j] = m_new;
      float sum = 0.f;
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const float p = exp2f(logit[f][j] - m_new);
        const int tile = f * TPC + (GQA == 4 ? (rq >> 1) : 0);
        L.p[hA + j][16 * tile + n] = p;
        sum += p;
      }
      l_part[j] = l_part[j] * alpha[j] + sum;
    }
    if (n == 0 && (GQA == 8 || rq < 2)) {
      L.alpha[hA] = alpha[0];
      L.alpha[hA + 1] = alpha[1];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value A operand: p s_t 2^(24-offset) 2^-E_V, hi/lo rows, via LDS
    float vs[8];
    float vmax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vs[e] = h2f(vsb[e]);
      vmax = fmaxf(vmax, vs[e]);
    }
    vmax = wave_max16(vmax);
    const int e_v_new = max(e_v, ceil_exp(vmax) + 9);
    const float vshift = exp2i(max(-126, min(127, e_v - e_v_new)));   // 0 on the first group
    const float sv = exp2i(max(-126, min(127, -e_v_new)));
    e_v = e_v_new;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int h = ph + 4 * j;
      const float al = L.alpha[h];
      float v[8];
      float mt = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = chunk_index<BITS>(pc, pkq, e);
        const float p = L.p[h][t];
        v[e] = p * vs[e] * exp2i(24 - code_offset<BITS>(t)) * sv;
        mt = fmaf(p, h2f(vmb[e]), mt);
      }
      mterm[j] = fmaf(mterm[j], al, mt);
      u32x4 hi, lo;
      split_hilo(v, hi, lo);
      L.av[pc][pkq][2 * h] = hi;
      L.av[pc][pkq][2 * h + 1] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- rescale the p.V accumulators (alpha and the exponent change)
    {
      const bool real_rows = GQA == 8 || rq < 2;
      const int h0 = GQA == 4 ? 2 * rq : 2 * rq;
      const float f0 = real_rows ? L.alpha[h0] * vshift : 0.f;
      const float f1 = real_rows ? L.alpha[h0 + 1] * vshift : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][0] *= f0;
        acc[i][1] *= f0;
        acc[i][2] *= f1;
        acc[i][3] *= f1;
      }
    }

    // ---- p.V
    u32x4 apv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      apv[c] = (m_row < 2 * GQA) ? L.av[c][kq][m_row] : sh.main.zero;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int e = blk >> 2, comp = blk & 3;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 bv;
        if (BITS == 2) {
          u32x4 q0, q1;
          conv2(vwords[c >> 1][e][comp], q0, q1);
          bv = (c & 1) ? q1 : q0;
        } else {
          bv = conv4(vwords[c][e][comp]);
        }
        acc[blk] = mfma(apv[c], bv, acc[blk]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---------------------------------------------------------------- merge waves
  // per-head totals of this wave
  float lsum[2], msave[2] = {m_run[0], m_run[1]};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float v = l_part[j];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    if (GQA == 4) v += __shfl_xor(v, 32);
    lsum[j] = v;
  }
  float mtsum[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    float v = mterm[j];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    mtsum[j] = v;
  }
  __syncthreads();   // the per-wave buffers are reused for the merge below
  MergeLds<GQA>& M = sh.merge;
  if (n == 0 && (GQA == 8 || rq < 2)) {
    M.m[wave][hA] = msave[0];
    M.m[wave][hA + 1] = msave[1];
    M.l[wave][hA] = lsum[0];
    M.l[wave][hA + 1] = lsum[1];
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < NH; ++j) M.mt[wave][ph + 4 * j] = mtsum[j];
  }
  __syncthreads();
  {
    const bool real_rows = GQA == 8 || rq < 2;
    if (real_rows) {
      const int h0 = 2 * rq;
      const float ev = exp2i(max(-126, min(127, e_v)));
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int d = 64 * (blk >> 2) + 4 * n + (blk & 3);
        M.num[wave][h0][d] = fmaf(acc[blk][0] + acc[blk][1], ev, M.mt[wave][h0]);
        M.num[wave][h0 + 1][d] = fmaf(acc[blk][2] + acc[blk][3], ev, M.mt[wave][h0 + 1]);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < GQA * kD; i += kThreadsM) {
    const int h = i / kD, d = i % kD;
    float mm = kNegInfM;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (M.l[w][h] > 0.f) mm = fmaxf(mm, M.m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (M.l[w][h] > 0.f) {
        const float f = exp2f(M.m[w][h] - mm);
        num = fmaf(M.num[w][h][d], f, num);
        den = fmaf(M.l[w][h], f, den);
      }
    float* wp = a.ws + (((b * a.H_q) + hk * GQA + h) * n_parts + chunk) * (kD + 2);
    wp[2 + d] = num;
    if (d == 0) {
      wp[0] = mm;
      wp[1] = den;
    }
  }
}

}  // namespace

bool mfma_decode_supported(int bits, int group, int gqa, int n_boost) {
  return group == kG && (gqa == 4 || gqa == 8) && n_boost == 0 && (bits == 2 || bits == 4);
}

hipError_t launch_decode_mfma(int bits, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_chunks + 1), (unsigned)(a.B * a.H_kv));
  if (bits == 2) {
    if (a.gqa == 4) decode_mfma_kernel<2, 4><<<grid, kThreadsM, 0, st>>>(a);
    else decode_mfma_kernel<2, 8><<<grid, kThreadsM, 0, st>>>(a);
  } else {
    if (a.gqa == 4) decode_mfma_kernel<4, 4><<<grid, kThreadsM, 0, st>>>(a);
    else decode_mfma_kernel<4, 8><<<grid, kThreadsM, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvq
