// Quantize + pack, and dequantize, for the low-bit KV cache.
//
// KIVI page, Step 1 (`quant_kcache`): per group mn = min, scale =
// (max - mn)/(2^bits - 1), code = round(clamp((x - mn)/scale, 0, 2^bits-1));
// keys per channel over G tokens, values per token over G channels.
// KIVI page, Step 2 (`pack_tensor`): 32/bits codes per word, least
// significant first.  Kitty page, sections 3.2 and 4.1: per key group the
// n_boost channels of largest range get 4-bit codes, split into the dense
// low-two-bit word, a compact word of high two bits and a channel index.
//
// Exactness contract: fp32 range, IEEE fp32 division (hipcc's correctly
// rounded division), fp16 scale rounded to nearest even, codes divide by the
// stored scale, clamp, then round half to even (v_rndne_f32); min/max by the
// total order -0 < +0.  No floating-point contraction in this file.

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t quant_code(float x, float mn, float s, float maxq) {
  if (s == 0.0f) return 0u;
  float y = (x - mn) / s;
  y = fminf(fmaxf(y, 0.0f), maxq);
  return (uint32_t)__builtin_rintf(y);
}

// One block quantizes one (head, group) of keys (blockIdx.y == 0) or values
// (blockIdx.y == 1).  The fp16 source tile [G][D] is staged in LDS.
template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  constexpr int FPI = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int WPT = kD / FPI;          // key words per token
  __shared__ uint16_t tile[G * kD];
  __shared__ float s_mn[kD];             // keys: per channel; values: per (token, chan group)
  __shared__ float s_sc[kD];
  __shared__ float s_mq[kD];             // keys: maxq of each channel (3 or 15 with boost)
  __shared__ float s_rng[kD];
  __shared__ int s_flag[kD];             // keys: channel is boosted (Kitty)
  __shared__ int s_chan_of_row[kD];
  __shared__ uint32_t s_red[2][kD];

  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t head = blk / a.n_groups;
  const int64_t gi = blk % a.n_groups;          // group index inside the source
  const int64_t g = a.first_group + gi;         // group index in the cache
  const bool is_v = blockIdx.y != 0;
  const uint16_t* src = (is_v ? a.v_src : a.k_src) + head * a.src_head_stride + gi * G * kD;

  // stage the tile: 16-byte loads
  {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* t4 = reinterpret_cast<uint4*>(tile);
    for (int i = tid; i < G * kD / 8; i += kThreads) t4[i] = s4[i];
  }
  __syncthreads();

  if (!is_v) {
    // ---- keys: min/max per channel over G tokens (two threads per channel)
    const int d = tid & (kD - 1), half = tid >> 7;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = half * (G / 2); j < (half + 1) * (G / 2); ++j) {
      const uint32_t k = order_key(tile[j * kD + d]);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    if (half) {
      s_red[0][d] = lo;
      s_red[1][d] = hi;
    }
    __syncthreads();
    const int nb = a.n_boost;
    if (!half) {
      lo = min(lo, s_red[0][d]);
      hi = max(hi, s_red[1][d]);
      const float mn = h2f(from_order_key(lo));
      const float mx = h2f(from_order_key(hi));
      s_mn[d] = mn;
      s_rng[d] = mx - mn;
    }
    __syncthreads();
    if (!half && nb > 0) {
      // Kitty: rank by range, ties to the lower channel
      const float r = s_rng[d];
      int rank = 0;
      for (int c = 0; c < kD; ++c) {
        const float rc = s_rng[c];
        rank += (rc > r) || (rc == r && c < d);
      }
      s_flag[d] = rank < nb;
    }
    __syncthreads();
    if (!half) {
      int row = nb;  // sentinel: not boosted
      if (nb > 0 && s_flag[d]) {
        row = 0;  // boosted rows ascend with the channel index
        for (int c = 0; c < d; ++c) row += s_flag[c];
      }
      const float maxq = (row < nb) ? 15.0f : (float)MASK;
      const uint16_t sh = f2h(s_rng[d] / maxq);
      const int64_t m_off = (head * (a.c.t_cap / G) + g) * kD + d;
      a.c.k_scale[m_off] = sh;
      a.c.k_min[m_off] = from_order_key(lo);
      if (nb > 0) a.c.k_bidx[m_off] = (uint8_t)row;
      s_sc[d] = h2f(sh);
      s_mq[d] = maxq;
      if (row < nb) s_chan_of_row[row] = d;
    }
    __syncthreads();
    // ---- codes, packed along channels: word (t, w) holds channels w*FPI + j
    uint32_t* kw = a.c.k_codes + (head * a.c.t_cap + g * G) * WPT;
    for (int i = tid; i < G * WPT; i += kThreads) {
      const int t = i / WPT, w = i % WPT;
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < FPI; ++j) {
        const int c = w * FPI + j;
        const uint32_t q = quant_code(h2f(tile[t * kD + c]), s_mn[c], s_sc[c], s_mq[c]);
        word |= (q & MASK) << (BITS * j);
      }
      kw[i] = word;
    }
    if (nb > 0) {
      // Kitty high two bits of the boosted rows, 16 rows per word
      const int hpt = nb / 16;
      uint32_t* hw = a.c.k_hi + (head * a.c.t_cap + g * G) * hpt;
      for (int i = tid; i < G * hpt; i += kThreads) {
        const int t = i / hpt, w = i % hpt;
        uint32_t word = 0u;
        for (int j = 0; j < 16; ++j) {
          const int c = s_chan_of_row[w * 16 + j];
          const uint32_t q = quant_code(h2f(tile[t * kD + c]), s_mn[c], s_sc[c], 15.0f);
          word |= (q >> 2) << (2 * j);
        }
        hw[i] = word;
      }
    }
  } else {
    // ---- values: per token, per channel group of G channels
    constexpr int NCG = kD / G;            // channel groups per token
    constexpr int PAIRS = G * NCG;         // (token, channel group) pairs == kD
    static_assert(PAIRS == kD, "one pair per LDS slot");
    const int p = tid >> 1, half = tid & 1;
    const int t = p / NCG, cg = p % NCG;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = half * (G / 2); j < (half + 1) * (G / 2); ++j) {
      const uint32_t k = order_key(tile[t * kD + cg * G + j]);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, 1));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, 1));
    if (!half) {
      const float mn = h2f(from_order_key(lo));
      const float mx = h2f(from_order_key(hi));
      const uint16_t sh = f2h((mx - mn) / (float)MASK);
      const int64_t m_off = (head * a.c.t_cap + g * G + t) * NCG + cg;
      a.c.v_scale[m_off] = sh;
      a.c.v_min[m_off] = from_order_key(lo);
      s_mn[p] = mn;
      s_sc[p] = h2f(sh);
    }
    __syncthreads();
    // codes, packed along tokens: word (w, d) holds tokens w*FPI + j
    uint32_t* vw = a.c.v_codes + (head * (a.c.t_cap / FPI) + g * (G / FPI)) * kD;
    for (int i = tid; i < (G / FPI) * kD; i += kThreads) {
      const int w = i / kD, d = i % kD;
      const int cgd = d / G;
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < FPI; ++j) {
        const int tt = w * FPI + j;
        const int pp = tt * NCG + cgd;
        const uint32_t q = quant_code(h2f(tile[tt * kD + d]), s_mn[pp], s_sc[pp], (float)MASK);
        word |= q << (BITS * j);
      }
      vw[i] = word;
    }
  }
}

// Dequantize: one thread per (token, channel) of keys and values.
template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs a) {
  constexpr int FPI = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t n_tok = a.n_groups * G;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.n_heads * n_tok * kD;
  if (idx >= total) return;
  const int d = (int)(idx % kD);
  const int64_t i = (idx / kD) % n_tok;
  const int64_t head = idx / (kD * n_tok);
  const int64_t t = a.first_group * G + i;
  const int64_t g = t / G;
  // key
  {
    const uint32_t w = a.c.k_codes[(head * a.c.t_cap + t) * (kD / FPI) + d / FPI];
    uint32_t q = (w >> (BITS * (d % FPI))) & MASK;
    const int64_t m_off = (head * (a.c.t_cap / G) + g) * kD + d;
    if (a.n_boost > 0) {
      const int r = a.c.k_bidx[m_off];
      if (r < a.n_boost) {
        const uint32_t hw = a.c.k_hi[(head * a.c.t_cap + t) * (a.n_boost / 16) + r / 16];
        q |= ((hw >> (2 * (r % 16))) & 3u) << 2;
      }
    }
    const float prod = (float)q * h2f(a.c.k_scale[m_off]);
    a.k_out[idx] = prod + h2f(a.c.k_min[m_off]);
  }
  // value
  {
    const uint32_t w = a.c.v_codes[(head * (a.c.t_cap / FPI) + t / FPI) * kD + d];
    const uint32_t q = (w >> (BITS * (t % FPI))) & MASK;
    const int64_t m_off = (head * a.c.t_cap + t) * (kD / G) + d / G;
    const float prod = (float)q * h2f(a.c.v_scale[m_off]);
    a.v_out[idx] = prod + h2f(a.c.v_min[m_off]);
  }
}

template <int BITS>
hipError_t quantize_bits(int group, const QuantArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_heads * a.n_groups), 2);
  switch (group) {
    case 32: quantize_kernel<BITS, 32><<<grid, kThreads, 0, s>>>(a); break;
    case 64: quantize_kernel<BITS, 64><<<grid, kThreads, 0, s>>>(a); break;
    case 128: quantize_kernel<BITS, 128><<<grid, kThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t dequantize_bits(int group, const DequantArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.n_heads * a.n_groups * group * kD;
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  switch (group) {
    case 32: dequantize_kernel<BITS, 32><<<grid, kThreads, 0, s>>>(a); break;
    case 64: dequantize_kernel<BITS, 64><<<grid, kThreads, 0, s>>>(a); break;
    case 128: dequantize_kernel<BITS, 128><<<grid, kThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int bits, int group, const QuantArgs& a, hipStream_t s) {
  if (a.n_groups == 0 || a.n_heads == 0) return hipSuccess;
  return bits == 2 ? quantize_bits<2>(group, a, s) : quantize_bits<4>(group, a, s);
}

hipError_t launch_dequantize(int bits, int group, const DequantArgs& a, hipStream_t s) {
  if (a.n_groups == 0 || a.n_heads == 0) return hipSuccess;
  return bits == 2 ? dequantize_bits<2>(group, a, s) : dequantize_bits<4>(group, a, s);
}

}  // namespace kvq
