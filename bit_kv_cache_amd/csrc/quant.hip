// Quantize + pack, and dequantize, for the low-bit KV cache.
//
// KIVI page, Step 1 (`quant_kcache`): per group mn = min, scale =
// (max - mn)/(2^bits - 1), code = round(clamp((x - mn)/scale, 0, 2^bits-1));
// keys per channel over G tokens, values per token over G channels.
// KIVI page, Step 2 (`pack_tensor`): 32/bits codes per word, least
// significant first.  Kitty page, sections 3.2 and 4.1: per key group the
// n_boost most important channels (largest range, or largest mean magnitude
// over the group's tokens) get 4-bit codes, split into the dense
// low-two-bit word, a compact word of high two bits and a channel index.
// Keys and values may use different widths (Kitty page, section 3.1: K2V4,
// K4V2): BITS is the key width, VB the value width.
//
// Exactness contract: fp32 range, IEEE fp32 division (hipcc's correctly
// rounded division), fp16 scale rounded to nearest even, codes divide by the
// stored scale, clamp, then round half to even (v_rndne_f32); min/max by the
// total order -0 < +0.  No floating-point contraction in this file.
//
// Work split: every (head, group) is cut into 4 key slices of 32 channels and
// up to 4 value slices of whole packed words of tokens, one block each, so a
// one-group append over 64 heads already fills the GPU.  Kitty keys need the ranking of all channels
// of a group, so with n_boost > 0 one block quantizes the whole key group.

#include "kvq_internal.h"
#include "quant_common.h"
#include "merge_common.h"
#include "append_common.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kSlices = 4;

// |x| of an fp16 value in units of 2^-24, exactly: a subnormal's fraction,
// or the significand (implicit bit set) shifted by the biased exponent - 1.
// A group's sum (at most 128 values below 2^40 units) fits 64 bits exactly,
// so it does not depend on the order of the additions.
__device__ __forceinline__ uint64_t mag_units(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, f = h & 0x3FFu;
  return e == 0 ? (uint64_t)f : (uint64_t)(f | 0x400u) << (e - 1);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v, int width) {
  for (int o = 1; o < width; o <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v, int width) {
  for (int o = 1; o < width; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Keys, channels [32*slice, 32*slice+32) of one group (plain KIVI).
template <int BITS, int G>
__device__ void quantize_keys_slice(const QuantArgs& a, int64_t head, int64_t gi, int slice) {
  constexpr int FPI = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int WPT = kD / FPI;          // key words per token
  constexpr int CH = kD / kSlices;       // 32 channels
  constexpr int SW = CH / FPI;           // words per token in this slice
  __shared__ uint16_t tile[G][CH + 2];   // +2: odd row pitch in dwords
  __shared__ uint32_t red[2][8][CH];
  __shared__ float s_mn[CH], s_sc[CH], s_rs[CH];
  const int tid = threadIdx.x;
  const int64_t gb = group_block(a.c, head, a.first_group + gi, G);   // the group's block (page)
  if (gb < 0) return;                     // a page outside the pool: nothing is written
  const uint16_t* src = a.k_src + head * a.src_head_stride + gi * G * kD + slice * CH;
  // stage: each row contributes 64 bytes (4 x 16 B)
  for (int i = tid; i < G * 4; i += kThreads) {
    const int t = i >> 2, q = i & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(src + t * kD + 8 * q);
    uint32_t* d = reinterpret_cast<uint32_t*>(&tile[t][8 * q]);
    d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w;
  }
  __syncthreads();
  // min/max per channel: 8 token parts of G/8
  {
    const int c = tid & (CH - 1), part = tid >> 5;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int t = part * (G / 8); t < (part + 1) * (G / 8); ++t) {
      const uint32_t k = order_key(tile[t][c]);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    red[0][part][c] = lo;
    red[1][part][c] = hi;
  }
  __syncthreads();
  if (tid < CH) {
    uint32_t lo = red[0][0][tid], hi = red[1][0][tid];
#pragma unroll
    for (int p = 1; p < 8; ++p) {
      lo = min(lo, red[0][p][tid]);
      hi = max(hi, red[1][p][tid]);
    }
    const float mn = h2f(from_order_key(lo));
    const float mx = h2f(from_order_key(hi));
    const uint16_t sh = f2h((mx - mn) / (float)MASK);
    const int64_t m_off = gb * kD + slice * CH + tid;
    a.c.k_scale[m_off] = sh;
    a.c.k_min[m_off] = from_order_key(lo);
    s_mn[tid] = mn;
    s_sc[tid] = h2f(sh);
    s_rs[tid] = 1.0f / h2f(sh);
  }
  __syncthreads();
  // codes, packed along channels: word (t, w) holds channels w*FPI + j
  uint32_t* kw = a.c.k_codes + gb * G * WPT + slice * SW;
  for (int i = tid; i < G * SW; i += kThreads) {
    const int t = i / SW, w = i % SW;
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < FPI; ++j) {
      const int c = w * FPI + j;
      word |= quant_code_rcp(h2f(tile[t][c]), s_mn[c], s_sc[c], s_rs[c], (float)MASK)
              << (BITS * j);
    }
    kw[t * WPT + w] = word;
  }
}

// Keys of one whole group with the Kitty boost (2-bit, n_boost > 0).
//  * min / max (and the sum of |x|) per channel: a thread takes a channel
//    pair over a quarter of the tokens;
//  * rank of each channel by range (or by the sum of |x|, the mean's order),
//    ties to the lower channel: two threads per channel, half the channels
//    each; a channel is boosted when fewer than n_boost channels precede it;
//  * boosted row of a channel = number of boosted channels below it (rows
//    ascend with the channel index), from the two waves' ballots;
//  * codes: thread (token t, word w) codes channels 16w..16w+15 of token t
//    from two 16-byte reads (the statistics of its 16 channels sit in
//    registers), writes the low two bits as the packed word and ORs the high
//    two bits of boosted channels into the token's high-bits words in LDS.
template <int G>
__device__ void quantize_keys_kitty(const QuantArgs& a, int64_t head, int64_t gi) {
  constexpr int BITS = 2, FPI = 16, WPT = kD / FPI;
  constexpr uint32_t MASK = 3u;
  __shared__ alignas(16) uint16_t tile[G * kD];
  __shared__ float s_mn[kD], s_sc[kD], s_rs[kD], s_mq[kD];
  __shared__ alignas(16) float s_rng[kD];
  __shared__ int s_row[kD], s_rank[2][kD];
  __shared__ uint32_t s_lo4[4][kD], s_hi4[4][kD];
  __shared__ alignas(16) uint64_t s_mag4[4][kD];   // sum of |x| per token quarter (units of 2^-24)
  __shared__ alignas(16) uint64_t s_mag[kD];
  __shared__ uint64_t s_ballot[2];
  __shared__ uint32_t s_hi[G * (kD / 16)];     // high-bits words [token][n_boost / 16]
  const int tid = threadIdx.x;
  const int64_t gb = group_block(a.c, head, a.first_group + gi, G);
  if (gb < 0) return;
  const int nb = a.n_boost, hpt = nb / 16;
  const uint16_t* src = a.k_src + head * a.src_head_stride + gi * G * kD;
  {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* t4 = reinterpret_cast<uint4*>(tile);
    for (int i = tid; i < G * kD / 8; i += kThreads) t4[i] = s4[i];
    for (int i = tid; i < G * hpt; i += kThreads) s_hi[i] = 0u;
  }
  __syncthreads();
  const int d = tid & (kD - 1), half = tid >> 7;
  const bool by_mag = a.boost_score != 0;
  {
    // channels 2 cp, 2 cp + 1 over tokens [32 qt, 32 qt + 32)
    const int cp = tid & 63, qt = tid >> 6;
    const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tile);
    uint32_t lo0 = 0xFFFFFFFFu, hi0 = 0u, lo1 = 0xFFFFFFFFu, hi1 = 0u;
    uint64_t mag0 = 0, mag1 = 0;
    for (int j = qt * (G / 4); j < (qt + 1) * (G / 4); ++j) {
      const uint32_t x = t32[j * (kD / 2) + cp];
      const uint16_t x0 = (uint16_t)(x & 0xFFFFu), x1 = (uint16_t)(x >> 16);
      lo0 = min(lo0, order_key(x0));
      hi0 = max(hi0, order_key(x0));
      lo1 = min(lo1, order_key(x1));
      hi1 = max(hi1, order_key(x1));
      if (by_mag) {
        mag0 += mag_units(x0);
        mag1 += mag_units(x1);
      }
    }
    s_lo4[qt][2 * cp] = lo0;
    s_hi4[qt][2 * cp] = hi0;
    s_lo4[qt][2 * cp + 1] = lo1;
    s_hi4[qt][2 * cp + 1] = hi1;
    s_mag4[qt][2 * cp] = mag0;
    s_mag4[qt][2 * cp + 1] = mag1;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  if (!half) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo = min(lo, s_lo4[q][d]);
      hi = max(hi, s_hi4[q][d]);
    }
    s_mag[d] = (s_mag4[0][d] + s_mag4[1][d]) + (s_mag4[2][d] + s_mag4[3][d]);
    const float mn = h2f(from_order_key(lo));
    s_mn[d] = mn;
    s_rng[d] = h2f(from_order_key(hi)) - mn;
  }
  __syncthreads();
  {
    // channels of this thread's half that rank before channel d
    int cnt = 0;
    const int c0 = half * (kD / 2);
    if (by_mag) {
      const uint64_t v = s_mag[d];
      const ulonglong2* m2 = reinterpret_cast<const ulonglong2*>(s_mag + c0);
      for (int c = 0; c < kD / 4; ++c) {
        const ulonglong2 vc = m2[c];
        const int ca = c0 + 2 * c;
        cnt += (vc.x > v) || (vc.x == v && ca < d);
        cnt += (vc.y > v) || (vc.y == v && ca + 1 < d);
      }
    } else {
      const float r = s_rng[d];
      const float4* r4 = reinterpret_cast<const float4*>(s_rng + c0);
      for (int c = 0; c < kD / 8; ++c) {
        const float4 rc = r4[c];
        const int ca = c0 + 4 * c;
        cnt += (rc.x > r) || (rc.x == r && ca < d);
        cnt += (rc.y > r) || (rc.y == r && ca + 1 < d);
        cnt += (rc.z > r) || (rc.z == r && ca + 2 < d);
        cnt += (rc.w > r) || (rc.w == r && ca + 3 < d);
      }
    }
    s_rank[half][d] = cnt;
  }
  __syncthreads();
  bool boosted = false;
  if (!half) {
    boosted = s_rank[0][d] + s_rank[1][d] < nb;
    const uint64_t m = __ballot(boosted);   // waves 0 and 1: channels 0..63, 64..127
    if ((tid & 63) == 0) s_ballot[tid >> 6] = m;
  }
  __syncthreads();
  if (!half) {
    int row = nb;  // sentinel: not boosted
    if (boosted) {
      const int bit = d & 63;
      const uint64_t below = bit ? (s_ballot[d >> 6] & ((1ull << bit) - 1ull)) : 0ull;
      row = __popcll(below) + (d >= 64 ? __popcll(s_ballot[0]) : 0);
    }
    const float maxq = (row < nb) ? 15.0f : (float)MASK;
    const uint16_t sh = f2h(s_rng[d] / maxq);
    const int64_t m_off = gb * kD + d;
    a.c.k_scale[m_off] = sh;
    a.c.k_min[m_off] = from_order_key(lo);
    a.c.k_bidx[m_off] = (uint8_t)row;
    s_sc[d] = h2f(sh);
    s_rs[d] = 1.0f / h2f(sh);
    s_mq[d] = maxq;
    s_row[d] = row;
  }
  __syncthreads();
  // every thread codes the same 16 channels (kThreads is a multiple of WPT)
  const int w = tid % WPT;
  float mn[FPI], sc[FPI], rs[FPI], mq[FPI];
  int rw[FPI];
#pragma unroll
  for (int j = 0; j < FPI; ++j) {
    const int c = w * FPI + j;
    mn[j] = s_mn[c];
    sc[j] = s_sc[c];
    rs[j] = s_rs[c];
    mq[j] = s_mq[c];
    rw[j] = s_row[c];
  }
  uint32_t* kw = a.c.k_codes + gb * G * WPT;
  for (int i = tid; i < G * WPT; i += kThreads) {
    const int t = i / WPT;
    const uint4* x4 = reinterpret_cast<const uint4*>(tile + t * kD + w * FPI);
    const uint4 x0 = x4[0], x1 = x4[1];
    const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < FPI; ++j) {
      const uint16_t xh = (uint16_t)(xs[j >> 1] >> (16 * (j & 1)));
      const uint32_t q = quant_code_rcp(h2f(xh), mn[j], sc[j], rs[j], mq[j]);
      word |= (q & MASK) << (BITS * j);
      if (rw[j] < nb)
        atomicOr(&s_hi[t * hpt + (rw[j] >> 4)], (q >> 2) << (2 * (rw[j] & 15)));
    }
    kw[i] = word;
  }
  __syncthreads();
  uint32_t* hw = a.c.k_hi + gb * G * hpt;
  for (int i = tid; i < G * hpt; i += kThreads) hw[i] = s_hi[i];
}

// Value slices per group: whole packed words (FPI tokens) per slice.
template <int BITS, int G>
constexpr int kValueSlices = (G / (32 / BITS)) < kSlices ? (G / (32 / BITS)) : kSlices;

// Values, tokens [slice*NT, (slice+1)*NT) of one group: per token, per
// channel group of G channels; codes packed along tokens.
template <int BITS, int G>
__device__ void quantize_values_slice(const QuantArgs& a, int64_t head, int64_t gi, int slice) {
  constexpr int FPI = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int NT = G / kValueSlices<BITS, G>;   // tokens in this slice (multiple of FPI)
  constexpr int NCG = kD / G;            // channel groups per token
  constexpr int TPP = kThreads / (NT * NCG);   // threads per (token, channel group)
  __shared__ uint16_t tile[NT][kD + 2];
  __shared__ float s_mn[NT * NCG], s_sc[NT * NCG], s_rs[NT * NCG];
  static_assert(FPI <= NT && NT % FPI == 0, "whole words per slice");
  static_assert(TPP >= 1 && (TPP & (TPP - 1)) == 0 && G % TPP == 0, "thread split");
  const int tid = threadIdx.x;
  const int64_t gb = group_block(a.c, head, a.first_group + gi, G);
  if (gb < 0) return;
  const int t_base = slice * NT;
  const uint16_t* src = a.v_src + head * a.src_head_stride + (gi * G + t_base) * kD;
  for (int i = tid; i < NT * kD / 8; i += kThreads) {
    const int t = i / (kD / 8), q = i % (kD / 8);
    const uint4 v = *reinterpret_cast<const uint4*>(src + t * kD + 8 * q);
    uint32_t* d = reinterpret_cast<uint32_t*>(&tile[t][8 * q]);
    d[0] = v.x, d[1] = v.y, d[2] = v.z, d[3] = v.w;
  }
  __syncthreads();
  {
    const int p = tid / TPP, part = tid % TPP;   // p = token * NCG + channel group
    const int t = p / NCG, cg = p % NCG;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = part * (G / TPP); j < (part + 1) * (G / TPP); ++j) {
      const uint32_t k = order_key(tile[t][cg * G + j]);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    lo = wave_min(lo, TPP);
    hi = wave_max(hi, TPP);
    if (part == 0) {
      const float mn = h2f(from_order_key(lo));
      const float mx = h2f(from_order_key(hi));
      const uint16_t sh = f2h((mx - mn) / (float)MASK);
      const int64_t m_off = (gb * G + t_base + t) * NCG + cg;
      a.c.v_scale[m_off] = sh;
      a.c.v_min[m_off] = from_order_key(lo);
      s_mn[p] = mn;
      s_sc[p] = h2f(sh);
      s_rs[p] = 1.0f / h2f(sh);
    }
  }
  __syncthreads();
  uint32_t* vw = a.c.v_codes + ((gb * G + t_base) / FPI) * kD;
  for (int i = tid; i < (NT / FPI) * kD; i += kThreads) {
    const int w = i / kD, d = i % kD;
    const int cgd = d / G;
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < FPI; ++j) {
      const int tt = w * FPI + j;
      const int pp = tt * NCG + cgd;
      word |= quant_code_rcp(h2f(tile[tt][d]), s_mn[pp], s_sc[pp], s_rs[pp], (float)MASK)
              << (BITS * j);
    }
    vw[i] = word;
  }
}

// grid: (heads * n_groups, 2 * kSlices): y < kSlices key slices (Kitty: the
// whole key group in y == 0), then value slices
template <int BITS, int VB, int G, bool KITTY>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  const int64_t blk = blockIdx.x;
  const int64_t head = blk / a.n_groups;
  const int64_t gi = blk % a.n_groups;
  const int y = blockIdx.y;
  if (y >= kSlices) {
    if (y - kSlices < kValueSlices<VB, G>) quantize_values_slice<VB, G>(a, head, gi, y - kSlices);
  } else if constexpr (KITTY) {
    if (y == 0) quantize_keys_kitty<G>(a, head, gi);
  } else {
    quantize_keys_slice<BITS, G>(a, head, gi, y);
  }
}

// The merge of a decode step and the quantize of the group it appends, in
// one launch: blocks [0, n_merge) merge two (batch, query head) rows each
// (threads 0..127 and 128..255, one channel per thread); the blocks after
// them are the quantize kernel's (group, slice) blocks.  The two jobs share
// no memory (partials and output vs. residual rows and one cache group).
template <int BITS, int VB, int G, bool KITTY, int NPM>
__global__ __launch_bounds__(kThreads) void merge_append_kernel(DecodeArgs d, QuantArgs a,
                                                               int n_merge) {
  const int blk = blockIdx.x;
  if (blk < n_merge) {
    const int64_t bh = 2 * (int64_t)blk + (threadIdx.x >> 7);
    if (bh < (int64_t)d.B * d.H_q) merge_row<NPM>(d.ws, d.n_parts, d.out, bh, threadIdx.x & 127);
    return;
  }
  const int qb = blk - n_merge;
  const int64_t head = qb / (2 * kSlices);   // one group: (head, slice)
  const int y = qb % (2 * kSlices);
  if (y >= kSlices) {
    if (y - kSlices < kValueSlices<VB, G>) quantize_values_slice<VB, G>(a, head, 0, y - kSlices);
  } else if constexpr (KITTY) {
    if (y == 0) quantize_keys_kitty<G>(a, head, 0);
  } else {
    quantize_keys_slice<BITS, G>(a, head, 0, y);
  }
}

// The merge of a decode step and the append of its full residual group as
// the split-K kernel's append items (append_common.h: 8 key items of 16
// channels and 8 value items of 16 tokens, each self-contained in one wave,
// with no LDS and no barrier): blocks [0, n_merge) merge 8 (batch, query
// head) rows each, one channel per thread; each block after them runs the 16
// items of one head, one per wave, so the stores of a head's group (each
// item writes part of the same cache lines) meet in one CU and one L2.
// Plain 2- or 4-bit codes of equal widths, G = 128.
template <int BITS, int NPM>
__global__ __launch_bounds__(1024) void merge_items_kernel(DecodeArgs d, int n_merge) {
  const int blk = blockIdx.x;
  if (blk < n_merge) {
    const int64_t bh = 8 * (int64_t)blk + (threadIdx.x >> 7);
    if (bh < (int64_t)d.B * d.H_q) merge_row<NPM>(d.ws, d.n_parts, d.out, bh, threadIdx.x & 127);
    return;
  }
  app::run_items<BITS, 1, true>(d, (int64_t)(blk - n_merge), (int)(threadIdx.x >> 6), app::kItems,
                          (int)(threadIdx.x & 63));
}

// Dequantize: one thread per (token, channel) of keys and values.
// The same for Kitty caches (2-bit codes with boosted key channels, G =
// 128, boosted channels ranked by range): each block after the merge rows
// runs one head's group as 16 waves, the 8 key items of the Kitty ranking
// (append_common.h, three barriers) and the 8 plain 2-bit value items.
template <int NPM>
__global__ __launch_bounds__(1024) void merge_kitty_items_kernel(DecodeArgs d, int n_merge) {
  __shared__ app::KittyLds s;
  const int blk = blockIdx.x;
  if (blk < n_merge) {
    const int64_t bh = 8 * (int64_t)blk + (threadIdx.x >> 7);
    if (bh < (int64_t)d.B * d.H_q) merge_row<NPM>(d.ws, d.n_parts, d.out, bh, threadIdx.x & 127);
    return;
  }
  const int64_t head = blk - n_merge;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t gb = group_block(d.c, head, d.n_groups, app::kG);
  if (gb < 0) return;   // a page outside the pool: the whole block writes nothing
  const int nb = d.n_boost, n_hi = app::kG * (nb >> 4);
  app::u32x4 x[4];
  app::item_load(d, head, wave, lane, x);
  if (tid < n_hi) s.hi[tid] = 0u;
  app::KittyKey k;
  if (wave < 8) app::kitty_stats(x, wave, lane, k, s);
  else app::item_store<2, true>(d, head, wave, lane, x);
  __syncthreads();
  if (wave < 8) app::kitty_rank(wave, lane, nb, s);
  __syncthreads();
  if (wave < 8) app::kitty_codes(d, gb, wave, lane, x, k, s, nb);
  __syncthreads();
  if (tid < n_hi) d.c.k_hi[gb * n_hi + tid] = s.hi[tid];
}

template <int BITS, int VB, int G>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs a) {
  constexpr int FPI = 32 / BITS, VFPI = 32 / VB;
  constexpr uint32_t MASK = (1u << BITS) - 1u, VMASK = (1u << VB) - 1u;
  const int64_t n_tok = a.n_groups * G;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.n_heads * n_tok * kD;
  if (idx >= total) return;
  const int d = (int)(idx % kD);
  const int64_t i = (idx / kD) % n_tok;
  const int64_t head = idx / (kD * n_tok);
  const int64_t t = a.first_group * G + i;
  const int64_t gb = group_block(a.c, head, t / G, G);
  if (gb < 0) {   // a page outside the pool
    a.k_out[idx] = a.v_out[idx] = __builtin_nanf("");
    return;
  }
  const int64_t tb = gb * G + t % G;   // the token's row in the block layout
  // key
  {
    const uint32_t w = a.c.k_codes[tb * (kD / FPI) + d / FPI];
    uint32_t q = (w >> (BITS * (d % FPI))) & MASK;
    const int64_t m_off = gb * kD + d;
    if (a.n_boost > 0) {
      const int r = a.c.k_bidx[m_off];
      if (r < a.n_boost) {
        const uint32_t hw = a.c.k_hi[tb * (a.n_boost / 16) + r / 16];
        q |= ((hw >> (2 * (r % 16))) & 3u) << 2;
      }
    }
    const float prod = (float)q * h2f(a.c.k_scale[m_off]);
    a.k_out[idx] = prod + h2f(a.c.k_min[m_off]);
  }
  // value
  {
    const uint32_t w = a.c.v_codes[(tb / VFPI) * kD + d];
    const uint32_t q = (w >> (VB * (t % VFPI))) & VMASK;
    const int64_t m_off = tb * (kD / G) + d / G;
    const float prod = (float)q * h2f(a.c.v_scale[m_off]);
    a.v_out[idx] = prod + h2f(a.c.v_min[m_off]);
  }
}

// Equal key and value widths are built for every group size, the mixed
// pairs (K2V4, K4V2) for G = 128 only.
template <int BITS, int VB, bool KITTY>
hipError_t quantize_bits(int group, const QuantArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_heads * a.n_groups), 2 * kSlices);
  if constexpr (VB != BITS) {
    if (group != 128) return hipErrorInvalidValue;
    quantize_kernel<BITS, VB, 128, KITTY><<<grid, kThreads, 0, s>>>(a);
  } else {
    switch (group) {
      case 32: quantize_kernel<BITS, VB, 32, KITTY><<<grid, kThreads, 0, s>>>(a); break;
      case 64: quantize_kernel<BITS, VB, 64, KITTY><<<grid, kThreads, 0, s>>>(a); break;
      case 128: quantize_kernel<BITS, VB, 128, KITTY><<<grid, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// Quantize + pack of whole groups as the decode step's append items
// (append_common.h: 8 key items of 16 channels and 8 value items of 16
// tokens, each in one wave, reading whole 32-byte pieces of the source rows
// and writing whole packed words).  Plain codes: four 4-wave blocks per
// (head, group), block j running items 4j..4j+3 (the key items of channels
// 0..63, of 64..127, the value items of tokens 0..63, of 64..127), so every
// 128-byte line of a group's rows is read by one block.  With KITTY (2-bit
// codes, 16 boosted channels ranked by range) one 16-wave block per (head,
// group), waves 0..7 running the Kitty key items, which meet in LDS three
// times.  The items' arithmetic is the quantize kernel's (quant_common.h),
// so the codes are the same bit for bit.  Equal widths, G = 128, a source
// head stride that is a whole number of rows.
template <int BITS, bool KITTY>
__global__ __launch_bounds__(KITTY ? 1024 : 256) void items_quantize_kernel(QuantArgs q) {
  __shared__ app::KittyLds ks;
  constexpr int kBlocksPerGroup = KITTY ? 1 : 4;
  const int64_t hg = blockIdx.x / kBlocksPerGroup;
  const int64_t head = hg / q.n_groups, gi = hg - head * q.n_groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (tid >> 6) + (KITTY ? 0 : 4 * (int)(blockIdx.x % kBlocksPerGroup));
  DecodeArgs d{};
  d.c = q.c;
  d.n_boost = q.n_boost;
  d.res_cap = (int32_t)(q.src_head_stride / kD);   // rows per source head
  d.k_res = q.k_src + gi * app::kG * kD;            // the group's first row of head 0
  d.v_res = q.v_src + gi * app::kG * kD;
  d.n_groups = q.first_group + gi;                  // the cache group the items write
  app::u32x4 x[4];
  app::item_load(d, head, wave, lane, x);
  if constexpr (KITTY) {
    const int64_t gb = group_block(d.c, head, d.n_groups, app::kG);
    if (gb < 0) return;   // a page outside the pool: the whole block writes nothing
    const int n_hi = app::kG * (q.n_boost >> 4);
    if (tid < n_hi) ks.hi[tid] = 0u;
    app::KittyKey k;
    if (wave < 8) app::kitty_stats(x, wave, lane, k, ks);
    else app::item_store<2, true>(d, head, wave, lane, x);
    __syncthreads();
    if (wave < 8) app::kitty_rank(wave, lane, q.n_boost, ks);
    __syncthreads();
    if (wave < 8) app::kitty_codes(d, gb, wave, lane, x, k, ks, q.n_boost);
    __syncthreads();
    if (tid < n_hi) d.c.k_hi[gb * n_hi + tid] = ks.hi[tid];
  } else {
    app::item_store<BITS, true>(d, head, wave, lane, x);
  }
}

template <int BITS, int VB>
hipError_t dequantize_bits(int group, const DequantArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.n_heads * a.n_groups * group * kD;
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  if constexpr (VB != BITS) {
    if (group != 128) return hipErrorInvalidValue;
    dequantize_kernel<BITS, VB, 128><<<grid, kThreads, 0, s>>>(a);
  } else {
    switch (group) {
      case 32: dequantize_kernel<BITS, VB, 32><<<grid, kThreads, 0, s>>>(a); break;
      case 64: dequantize_kernel<BITS, VB, 64><<<grid, kThreads, 0, s>>>(a); break;
      case 128: dequantize_kernel<BITS, VB, 128><<<grid, kThreads, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int BITS, int VB, bool KITTY, int NPM>
hipError_t merge_append_bits(int group, const DecodeArgs& d, const QuantArgs& a, hipStream_t s) {
  const int n_merge = (int)(((int64_t)d.B * d.H_q + 1) / 2);
  const dim3 grid((unsigned)(n_merge + a.n_heads * 2 * kSlices));
  if constexpr (VB != BITS) {
    if (group != 128) return hipErrorInvalidValue;
    merge_append_kernel<BITS, VB, 128, KITTY, NPM><<<grid, kThreads, 0, s>>>(d, a, n_merge);
  } else {
    switch (group) {
      case 32: merge_append_kernel<BITS, VB, 32, KITTY, NPM><<<grid, kThreads, 0, s>>>(d, a, n_merge); break;
      case 64: merge_append_kernel<BITS, VB, 64, KITTY, NPM><<<grid, kThreads, 0, s>>>(d, a, n_merge); break;
      case 128: merge_append_kernel<BITS, VB, 128, KITTY, NPM><<<grid, kThreads, 0, s>>>(d, a, n_merge); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int BITS, int NPM>
hipError_t merge_items_bits(const DecodeArgs& d, hipStream_t s) {
  const int n_merge = (int)(((int64_t)d.B * d.H_q + 7) / 8);
  const dim3 grid((unsigned)(n_merge + (int64_t)d.B * d.H_kv));
  merge_items_kernel<BITS, NPM><<<grid, 1024, 0, s>>>(d, n_merge);
  return hipGetLastError();
}

template <int NPM>
hipError_t merge_kitty_items(const DecodeArgs& d, hipStream_t s) {
  const int n_merge = (int)(((int64_t)d.B * d.H_q + 7) / 8);
  const dim3 grid((unsigned)(n_merge + (int64_t)d.B * d.H_kv));
  merge_kitty_items_kernel<NPM><<<grid, 1024, 0, s>>>(d, n_merge);
  return hipGetLastError();
}

template <int BITS, int VB, bool KITTY>
hipError_t merge_append_parts(int group, const DecodeArgs& d, const QuantArgs& a, hipStream_t s) {
  if (d.n_parts <= 8) return merge_append_bits<BITS, VB, KITTY, 8>(group, d, a, s);
  if (d.n_parts <= 16) return merge_append_bits<BITS, VB, KITTY, 16>(group, d, a, s);
  return merge_append_bits<BITS, VB, KITTY, kMergeAppendParts>(group, d, a, s);
}

}  // namespace

hipError_t launch_merge_append(int bits, int v_bits, int group, const DecodeArgs& d,
                               const QuantArgs& a, hipStream_t s) {
  if (d.n_parts > kMergeAppendParts || a.n_groups != 1) {
    const hipError_t e = launch_merge(d, s);
    return e != hipSuccess ? e : launch_quantize(bits, v_bits, group, a, s);
  }
  if (bits == v_bits && (bits == 2 || bits == 4) && group == 128 && a.n_boost == 0 &&
      d.n_parts <= 16 && d.res_cap >= 128) {
    // the merge and the append's items (one item per wave, no barriers)
    if (bits == 2)
      return d.n_parts <= 8 ? merge_items_bits<2, 8>(d, s) : merge_items_bits<2, 16>(d, s);
    return d.n_parts <= 8 ? merge_items_bits<4, 8>(d, s) : merge_items_bits<4, 16>(d, s);
  }
  if (bits == 2 && v_bits == 2 && group == 128 && a.n_boost > 0 && a.n_boost == d.n_boost &&
      a.boost_score == 0 && d.n_parts <= 16 && d.res_cap >= 128)
    return d.n_parts <= 8 ? merge_kitty_items<8>(d, s) : merge_kitty_items<16>(d, s);
  if (bits == 2 && v_bits == 4) return merge_append_parts<2, 4, false>(group, d, a, s);
  if (bits == 4 && v_bits == 2) return merge_append_parts<4, 2, false>(group, d, a, s);
  if (bits != v_bits) return hipErrorInvalidValue;
  if (bits == 2)
    return a.n_boost > 0 ? merge_append_parts<2, 2, true>(group, d, a, s)
                         : merge_append_parts<2, 2, false>(group, d, a, s);
  if (bits == 8) return merge_append_parts<8, 8, false>(group, d, a, s);
  return merge_append_parts<4, 4, false>(group, d, a, s);
}

hipError_t launch_quantize(int bits, int v_bits, int group, const QuantArgs& a, hipStream_t s) {
  if (a.n_groups == 0 || a.n_heads == 0) return hipSuccess;
  if (bits == v_bits && group == 128 && a.src_head_stride % kD == 0 &&
      a.src_head_stride / kD <= INT32_MAX && 4 * (int64_t)a.n_heads * a.n_groups <= INT32_MAX) {
    const int64_t groups = (int64_t)a.n_heads * a.n_groups;
    const dim3 grid4((unsigned)(4 * groups)), grid1((unsigned)groups);
    if (bits == 2 && a.n_boost == 0) {
      items_quantize_kernel<2, false><<<grid4, 256, 0, s>>>(a);
      return hipGetLastError();
    }
    if (bits == 4 && a.n_boost == 0) {
      items_quantize_kernel<4, false><<<grid4, 256, 0, s>>>(a);
      return hipGetLastError();
    }
    if (bits == 2 && a.n_boost == 16 && a.boost_score == 0) {
      items_quantize_kernel<2, true><<<grid1, 1024, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  if (bits == 2 && v_bits == 4) return quantize_bits<2, 4, false>(group, a, s);
  if (bits == 4 && v_bits == 2) return quantize_bits<4, 2, false>(group, a, s);
  if (bits != v_bits) return hipErrorInvalidValue;
  if (bits == 2)
    return a.n_boost > 0 ? quantize_bits<2, 2, true>(group, a, s)
                         : quantize_bits<2, 2, false>(group, a, s);
  if (bits == 8) return quantize_bits<8, 8, false>(group, a, s);
  return quantize_bits<4, 4, false>(group, a, s);
}

hipError_t launch_dequantize(int bits, int v_bits, int group, const DequantArgs& a,
                             hipStream_t s) {
  if (a.n_groups == 0 || a.n_heads == 0) return hipSuccess;
  if (bits == 2 && v_bits == 4) return dequantize_bits<2, 4>(group, a, s);
  if (bits == 4 && v_bits == 2) return dequantize_bits<4, 2>(group, a, s);
  if (bits != v_bits) return hipErrorInvalidValue;
  if (bits == 8) return dequantize_bits<8, 8>(group, a, s);
  return bits == 2 ? dequantize_bits<2, 2>(group, a, s) : dequantize_bits<4, 4>(group, a, s);
}

}  // namespace kvq
