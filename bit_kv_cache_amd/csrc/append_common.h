// The append of a decode step, run inside the decode kernels (not
// installed): the quantize + pack of the G = 128 rows of the residual window
// that has filled up (rows 0..127 of the head's residual buffer) into cache
// group n_groups, with the arithmetic of the quantize kernel (KIVI page,
// Steps 1-2): min and max by the total order -0 < +0, scale
// fp16((max - min) / maxq), codes as quant_code_rcp gives them, least significant code
// first.  The codes are bit-identical to kvq_quantize_pack's.
//
// The group is cut into 16 self-contained items: items 0..7 are key channels
// 16k..16k+15 over the 128 tokens (per-channel statistics), items 8..15 value
// tokens 16(k-8)..16(k-8)+15 over the 128 channels (per-token statistics).
// Each item writes whole packed words: keys are packed along channels (16 or
// 8 codes per word), values along tokens.  The appended group lies past
// every group the decode reads.
//
// Lane layout of an item's 4 x 8 fp16 inputs: keys, lane l holds tokens
// l/2 + 32i (i < 4) and channels c0 + 8(l%2) .. + 7; values, tokens
// t0 + l/16 + 4i and channels 8(l%16) .. + 7.
#pragma once

#include "quant_common.h"

namespace kvq {
namespace app {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kItems = 16;
constexpr int kG = 128;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Order keys (order_key) of the two fp16 values of a word, side by side: an
// fp16 value h maps to h XOR 0xFFFF when negative and h XOR 0x8000
// otherwise, which orders -0 < +0 and every finite value as its number.
__device__ __forceinline__ uint32_t order_keys2(uint32_t w) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  // each half's sign bit spread over the half (0xFFFF when negative)
  const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (short)15);
  return w ^ (m | 0x80008000u);
}
// min / max of two words of side-by-side 16-bit keys (packed integer ops)
__device__ __forceinline__ uint32_t min2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t max2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int e) {
  return (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
}

// A lane of the same row of 16 lanes (DPP): row rotations by 8 and 4, and
// the quad swaps of lanes 2 and 1 apart.
template <int CTRL>
__device__ __forceinline__ uint32_t row_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4E, kXor1 = 0xB1;

__device__ __forceinline__ void item_load(const DecodeArgs& a, int64_t head, int item, int lane,
                                          u32x4 (&x)[4]) {
  if (item < 8) {
    const uint16_t* src = a.k_res + head * a.res_cap * kD + 16 * item + 8 * (lane & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = *reinterpret_cast<const u32x4*>(src + ((lane >> 1) + 32 * i) * kD);
  } else {
    const uint16_t* src =
        a.v_res + (head * a.res_cap + 16 * (item - 8) + (lane >> 4)) * kD + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const u32x4*>(src + 4 * i * kD);
  }
}

// Code of x in a group (mn, s, rs) as quant_code_rcp computes it.  quot() is
// the quotient by the reciprocal, or (exact) by the IEEE division; the code
// is rint of the quotient clamped to maxq.  An item first codes every value
// by the reciprocal and notes whether any value of the wave lies within
// quant_code_rcp's tie window (|y - rint(y)| > 1/2 - 2^-16, both differences
// exact); only then does it code the item again by the IEEE quotient, so the
// window costs no branch per value (ONE_CHECK; otherwise quant_code_rcp
// itself, value by value, which keeps fewer registers live).  Outside the
// window both quotients give the same code, so the codes are
// quant_code_rcp's either way.  Clamping before rounding gives the same code
// (the bound is an integer), and a clamped quotient is never in the window
// unless the unclamped one is.  The groups' reciprocals are 0 for a zero
// scale (group_stat), so the quotient is 0 there and the code 0, the guard,
// with no select per value; x >= mn makes every quotient >= 0, so only the
// upper clamp remains.
//
// x is half `hi` of the fp16 word w; x - mn is taken by one v_fma_mix_f32
// (x converted exactly, times 1, minus mn, rounded once): the value of the
// fp32 subtraction, without a conversion of its own.
__device__ __forceinline__ float quot(uint32_t w, bool hi, float mn, float s, float rs,
                                      bool exact) {
#pragma clang fp contract(off)
  float d;
  if (hi)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(mn));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(mn));
  return exact ? (s == 0.0f ? 0.0f : d / s) : d * rs;
}

// Rounding by the magic number 1.5 * 2^23: for 0 <= yc <= 15, yc + 1.5 * 2^23
// lies in [2^23, 2^24), where the float spacing is 1, so the addition
// rounds yc to the nearest integer, ties to even (the even last mantissa
// bit), and the sum's bits are kRoundMagicBits + rint(yc).  Codes packed as
// sums of such bits, each shifted to its field, carry a constant
// (magic_sum) that one subtraction per word removes.  dev keeps the
// largest |yc - rint(yc)| (exact), tested against the window once.
constexpr float kRoundMagic = 12582912.0f;
constexpr uint32_t kRoundMagicBits = 0x4B400000u;
constexpr uint32_t magic_sum(int step, int n) {
  uint32_t s = 0u;
  for (int k = 0; k < n; ++k) s += kRoundMagicBits << (step * k);
  return s;
}
__device__ __forceinline__ uint32_t round_bits(float yc, float& dev) {
#pragma clang fp contract(off)
  const float t = yc + kRoundMagic;
  dev = fmaxf(dev, __builtin_fabsf(yc - (t - kRoundMagic)));
  return __builtin_bit_cast(uint32_t, t);
}
constexpr float kTieWindow = 0.5f - 0x1p-16f;   // near a tie: dev above this

// Scale and minimum of a group from the order keys of its extrema: pk holds
// the fp16 minimum (low half) and scale (high half), rs the scale's
// reciprocal (v_rcp_f32, within an ulp: enough for quant_code_rcp), or 0
// for a zero scale.
__device__ __forceinline__ void group_stat(uint32_t lo_key, uint32_t hi_key, float maxq,
                                           uint32_t& pk, float& rs) {
  const uint16_t l16 = from_order_key(lo_key);
  const uint16_t sh = group_scale(h2f(l16), h2f(from_order_key(hi_key)), maxq);
  const float sc = h2f(sh);
  rs = sc == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sc);
  pk = (uint32_t)l16 | ((uint32_t)sh << 16);
}
// The statistics (group_stat) that lane `src` computed, fetched by every
// lane: minimum and scale as floats, the reciprocal, and the packed halves.
__device__ __forceinline__ void fetch_stat(int src, uint32_t pk, float rs, uint32_t& pk_out,
                                           float& mn_out, float& sc_out, float& rs_out) {
  pk_out = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)pk);
  rs_out = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src,
                                                                  __builtin_bit_cast(int, rs)));
  mn_out = h2f((uint16_t)(pk_out & 0xFFFFu));
  sc_out = h2f((uint16_t)(pk_out >> 16));
}

// Minimum and maximum, as order keys, of the 8 channels c0 + 8(l%2) + e of a
// key item over its 128 tokens (lane layout above): order keys of channel
// pairs (2p, 2p + 1) side by side, over the lane's 4 tokens, the 8 lanes of
// its row with the same l%2 (DPP), then the four rows.  Every lane with the
// same l%2 ends with the same values.
__device__ __forceinline__ void key_extrema(const u32x4 (&x)[4], uint32_t (&lo)[8],
                                            uint32_t (&hi)[8]) {
  uint32_t lo2[4], hi2[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    lo2[p] = hi2[p] = order_keys2(x[0][p]);
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const uint32_t k = order_keys2(x[i][p]);
      lo2[p] = min2(lo2[p], k);
      hi2[p] = max2(hi2[p], k);
    }
    lo2[p] = min2(lo2[p], row_lane<kRor8>(lo2[p]));
    hi2[p] = max2(hi2[p], row_lane<kRor8>(hi2[p]));
    lo2[p] = min2(lo2[p], row_lane<kRor4>(lo2[p]));
    hi2[p] = max2(hi2[p], row_lane<kRor4>(hi2[p]));
    lo2[p] = min2(lo2[p], row_lane<kXor2>(lo2[p]));
    hi2[p] = max2(hi2[p], row_lane<kXor2>(hi2[p]));
  }
#pragma unroll
  for (int o = 16; o < 64; o <<= 1)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      lo2[p] = min2(lo2[p], (uint32_t)__shfl_xor((int)lo2[p], o));
      hi2[p] = max2(hi2[p], (uint32_t)__shfl_xor((int)hi2[p], o));
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = (lo2[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    hi[e] = (hi2[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  }
}

template <int BITS, bool ONE_CHECK>
__device__ __forceinline__ void item_store(const DecodeArgs& a, int64_t head, int item, int lane,
                                           const u32x4 (&x)[4]) {
  static_assert(BITS == 2 || BITS == 4, "2- or 4-bit codes");
  constexpr float kMaxq = (float)((1 << BITS) - 1);
  constexpr int kFpi = 32 / BITS;        // codes per word
  constexpr int kWpt = kD / kFpi;        // key words per token
  const int64_t blk = group_block(a.c, head, a.n_groups, kG);   // the appended group's block
  if (blk < 0) return;   // a page outside the pool: nothing is written
  if (item < 8) {
    const int c0 = 16 * item, q = lane & 1;
    uint32_t lo[8], hi[8];
    key_extrema(x, lo, hi);
    float mn[8], sc[8], rs[8];
    uint32_t pk[8];
    if constexpr (ONE_CHECK) {
      // Statistics one channel per lane: lane l takes channel c0 + 8q + es,
      // es = (l/2)%8 (lanes 16 apart repeat it), then every lane fetches its 8
      // channels' from lanes 2e + q of its row.
      const int es = (lane >> 1) & 7;
      uint32_t los = lo[0], his = hi[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        los = es == e ? lo[e] : los;
        his = es == e ? hi[e] : his;
      }
      uint32_t pk0;
      float rs0;
      group_stat(los, his, kMaxq, pk0, rs0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        fetch_stat((lane & 48) + 2 * e + q, pk0, rs0, pk[e], mn[e], sc[e], rs[e]);
    } else {
      // every lane its own 8 (no LDS traffic: this form runs beside the
      // decode's LDS ring)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        group_stat(lo[e], hi[e], kMaxq, pk[e], rs[e]);
        mn[e] = h2f((uint16_t)(pk[e] & 0xFFFFu));
        sc[e] = h2f((uint16_t)(pk[e] >> 16));
      }
    }
    if (lane < 2) {
      const int64_t m_off = blk * kD + c0 + 8 * q;
      u32x4 shw, mnw;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        shw[k] = __builtin_amdgcn_perm(pk[2 * k + 1], pk[2 * k], 0x07060302u);
        mnw[k] = __builtin_amdgcn_perm(pk[2 * k + 1], pk[2 * k], 0x05040100u);
      }
      *reinterpret_cast<u32x4*>(a.c.k_scale + m_off) = shw;
      *reinterpret_cast<u32x4*>(a.c.k_min + m_off) = mnw;
    }
    // codes of token t: channel c0 + 8q + e at bits BITS (c0 + 8q + e) mod
    // 32 of key word (c0 + 8q + e) / kFpi
    uint32_t parts[4];
    bool near = false;
    auto pack = [&](bool exact) {
      float dev = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t acc = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (ONE_CHECK) {
            const float y = quot(x[i][e >> 1], e & 1, mn[e], sc[e], rs[e], exact);
            acc += round_bits(fminf(y, kMaxq), dev) << (BITS * e);
          } else {
            const float xv = h2f(half_of(x[i], e));
            acc |= quant_code_rcp(xv, mn[e], sc[e], rs[e], kMaxq) << (BITS * e);
          }
        }
        if constexpr (ONE_CHECK) acc -= magic_sum(BITS, 8);
        // (8q + e) mod kFpi is e (4-bit) or 8q + e (2-bit)
        parts[i] = BITS == 2 ? acc << (16 * q) : acc;
      }
      if (!exact) near = dev > kTieWindow;
    };
    pack(false);
    if (ONE_CHECK && __any(near)) pack(true);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = (lane >> 1) + 32 * i;
      const uint32_t part = parts[i];
      if constexpr (BITS == 2) {
        // the two lanes of a token hold the two halves of one word
        const uint32_t word = part | row_lane<kXor1>(part);
        if (q == 0) a.c.k_codes[(blk * kG + t) * kWpt + item] = word;
      } else {
        a.c.k_codes[(blk * kG + t) * kWpt + 2 * item + q] = part;
      }
    }
  } else {
    const int t0 = 16 * (item - 8), r = lane >> 4, q = lane & 15;
    // per token over the 128 channels, as order keys of token pairs
    // (2u, 2u + 1) side by side: the lane's 8 channels (two per word, then
    // the word's halves), then the 16 lanes of the row (DPP)
    uint32_t lo2[2], hi2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t ml[2], mh[2];   // token 2u + k: even channels low, odd high
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4& v = x[2 * u + k];
        const uint32_t k0 = order_keys2(v[0]), k1 = order_keys2(v[1]);
        const uint32_t k2 = order_keys2(v[2]), k3 = order_keys2(v[3]);
        ml[k] = min2(min2(k0, k1), min2(k2, k3));
        mh[k] = max2(max2(k0, k1), max2(k2, k3));
      }
      lo2[u] = min2(__builtin_amdgcn_perm(ml[1], ml[0], 0x05040100u),
                    __builtin_amdgcn_perm(ml[1], ml[0], 0x07060302u));
      hi2[u] = max2(__builtin_amdgcn_perm(mh[1], mh[0], 0x05040100u),
                    __builtin_amdgcn_perm(mh[1], mh[0], 0x07060302u));
      lo2[u] = min2(lo2[u], row_lane<kRor8>(lo2[u]));
      hi2[u] = max2(hi2[u], row_lane<kRor8>(hi2[u]));
      lo2[u] = min2(lo2[u], row_lane<kRor4>(lo2[u]));
      hi2[u] = max2(hi2[u], row_lane<kRor4>(hi2[u]));
      lo2[u] = min2(lo2[u], row_lane<kXor2>(lo2[u]));
      hi2[u] = max2(hi2[u], row_lane<kXor2>(hi2[u]));
      lo2[u] = min2(lo2[u], row_lane<kXor1>(lo2[u]));
      hi2[u] = max2(hi2[u], row_lane<kXor1>(hi2[u]));
    }
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = (lo2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      hi[i] = (hi2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    }
    float mn[4], sc[4], rs[4];
    if constexpr (ONE_CHECK) {
      // Statistics one token per lane: lane l takes token t0 + r + 4 is, is =
      // l%4 (every 4 lanes of the row repeat them), stores them from the
      // first four lanes of its row, and every lane fetches its 4 tokens'
      // from lanes 16r + i.
      const int is = lane & 3;
      uint32_t los = lo[0], his = hi[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        los = is == i ? lo[i] : los;
        his = is == i ? hi[i] : his;
      }
      uint32_t pk0;
      float rs0;
      group_stat(los, his, kMaxq, pk0, rs0);
      if (q < 4) {
        const int64_t m_off = blk * kG + t0 + r + 4 * is;
        a.c.v_scale[m_off] = (uint16_t)(pk0 >> 16);
        a.c.v_min[m_off] = (uint16_t)(pk0 & 0xFFFFu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pk;
        fetch_stat((lane & 48) + i, pk0, rs0, pk, mn[i], sc[i], rs[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pk;
        group_stat(lo[i], hi[i], kMaxq, pk, rs[i]);
        mn[i] = h2f((uint16_t)(pk & 0xFFFFu));
        sc[i] = h2f((uint16_t)(pk >> 16));
        if (q == 0) {
          const int64_t m_off = blk * kG + t0 + r + 4 * i;
          a.c.v_scale[m_off] = (uint16_t)(pk >> 16);
          a.c.v_min[m_off] = (uint16_t)(pk & 0xFFFFu);
        }
      }
    }
    // codes: token t0 + j (j = r + 4i) at bits BITS (j mod kFpi) of word row
    // (t0 + j) / kFpi of its channel; the 4 lanes with the same q hold the
    // item's 16 tokens of a channel
    constexpr int kRows = 16 / kFpi;   // word rows of the item (1 or 2)
    uint32_t part[8][kRows];           // this lane's codes of channel 8q + e
    bool near = false;
    auto pack = [&](bool exact) {
      float dev = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t acc[kRows];
#pragma unroll
        for (int w = 0; w < kRows; ++w) acc[w] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // token j = r + 4i (i a compile-time index, r < 4): word row
          // (4 i) / kFpi, field j mod kFpi = r + (4 i) mod kFpi
          const int sh = BITS * ((4 * i) % kFpi);
          if constexpr (ONE_CHECK) {
            const float y = quot(x[i][e >> 1], e & 1, mn[i], sc[i], rs[i], exact);
            acc[(4 * i) / kFpi] += round_bits(fminf(y, kMaxq), dev) << sh;
          } else {
            const float xv = h2f(half_of(x[i], e));
            acc[(4 * i) / kFpi] |= quant_code_rcp(xv, mn[i], sc[i], rs[i], kMaxq) << sh;
          }
        }
#pragma unroll
        for (int w = 0; w < kRows; ++w) {
          if constexpr (ONE_CHECK) acc[w] -= magic_sum(4 * BITS, 4 / kRows);
          part[e][w] = acc[w] << (BITS * r);
        }
      }
      if (!exact) near = dev > kTieWindow;
    };
    pack(false);
    if (ONE_CHECK && __any(near)) pack(true);
    uint32_t wd[kRows][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int w = 0; w < kRows; ++w) {
        uint32_t p = part[e][w] | (uint32_t)__shfl_xor((int)part[e][w], 16);
        wd[w][e] = p | (uint32_t)__shfl_xor((int)p, 32);
      }
    }
    if (r == 0) {
#pragma unroll
      for (int w = 0; w < kRows; ++w) {
        uint32_t* dst = a.c.v_codes + (blk * (kG / kFpi) + t0 / kFpi + w) * kD + 8 * q;
        *reinterpret_cast<u32x4*>(dst) = u32x4{wd[w][0], wd[w][1], wd[w][2], wd[w][3]};
        *reinterpret_cast<u32x4*>(dst + 4) = u32x4{wd[w][4], wd[w][5], wd[w][6], wd[w][7]};
      }
    }
  }
}

// The items of slot `slot` among n_slots (slot = the calling wave's index
// among the waves of all the head's blocks that take items): slot, slot +
// n_slots, ... (n_slots >= 16 / MAXI).  Every item's inputs are requested
// before any is computed, so the wave waits for memory once.  Unrolled with
// guards: a loop here kept registers live into the decode loop and spilled.
template <int BITS, int MAXI, bool ONE_CHECK = false>
__device__ __forceinline__ void run_items(const DecodeArgs& a, int64_t head, int slot,
                                          int n_slots, int lane) {
  u32x4 x[MAXI][4];
#pragma unroll
  for (int k = 0; k < MAXI; ++k)
    if (slot + k * n_slots < kItems) item_load(a, head, slot + k * n_slots, lane, x[k]);
#pragma unroll
  for (int k = 0; k < MAXI; ++k)
    if (slot + k * n_slots < kItems)
      item_store<BITS, ONE_CHECK>(a, head, slot + k * n_slots, lane, x[k]);
}

// ------------------------------------------------------------ Kitty key items
//
// The Kitty page's key groups with boosted channels (sections 3.2 and 4.1):
// the n_boost channels of largest range (ties to the lower channel) take
// 4-bit codes, split into the low two bits in the dense 2-bit word and the
// high two bits in a compact word per token (boosted row r at bits 2(r%16)
// of word r/16, rows ascending with the channel), and k_bidx names each
// channel's row (n_boost: not boosted).  The 8 key items of a group run in
// the waves of one block and meet in LDS three times: their channels'
// ranges (kitty_stats), the boosted channels of each item (kitty_rank), and
// the high-bits words, which collect bits from every item (kitty_codes).
// Scales, minima and codes follow the quantize kernel's arithmetic.
struct KittyLds {
  alignas(16) float rng[kD];         // range (max - min in fp32) of every channel
  uint32_t bmask[8];                 // item w: bit j set when channel 16w + j is boosted
  uint32_t hi[kG * (kD / 16)];       // high-bits words [token][n_boost / 16]
};
struct KittyKey {
  uint32_t lo[8];                    // order keys of the minima of the lane's 8 channels
  float mn[8], rng[8];
};

// Extrema and ranges of the item's channels (the lane's 8: c0 + 8(l%2) + e);
// lanes 0 and 1 put the ranges in LDS.
__device__ __forceinline__ void kitty_stats(const u32x4 (&x)[4], int item, int lane,
                                            KittyKey& k, KittyLds& s) {
#pragma clang fp contract(off)
  uint32_t hi[8];
  key_extrema(x, k.lo, hi);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    k.mn[e] = h2f(from_order_key(k.lo[e]));
    k.rng[e] = h2f(from_order_key(hi[e])) - k.mn[e];
  }
  if (lane < 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s.rng[16 * item + 8 * lane + e] = k.rng[e];
  }
}

// Rank of each of the item's 16 channels among all 128 (channels with a
// larger range, or an equal one and a lower index): lane l counts channel
// 16 item + l%16 against channels 32(l/16) .. +31, the four counts add up
// over the lanes 16 apart; lane 0 puts the item's boosted set in LDS.
__device__ __forceinline__ void kitty_rank(int item, int lane, int n_boost, KittyLds& s) {
  const int d = 16 * item + (lane & 15), part = lane >> 4;
  const float r = s.rng[d];
  const float4* r4 = reinterpret_cast<const float4*>(s.rng + 32 * part);
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float4 rc = r4[c];
    const int ca = 32 * part + 4 * c;
    cnt += (rc.x > r) || (rc.x == r && ca < d);
    cnt += (rc.y > r) || (rc.y == r && ca + 1 < d);
    cnt += (rc.z > r) || (rc.z == r && ca + 2 < d);
    cnt += (rc.w > r) || (rc.w == r && ca + 3 < d);
  }
  cnt += __shfl_xor(cnt, 16);
  cnt += __shfl_xor(cnt, 32);
  const uint64_t m = __ballot(cnt < n_boost);
  if (lane == 0) s.bmask[item] = (uint32_t)(m & 0xFFFFu);
}

// Scales, minima, indices and codes of the item's channels in cache block
// blk: the dense words go to memory, the high two bits of boosted codes are
// ORed into the LDS words (each bit pair has one writer; the block stores
// the words after its next barrier).  Codes as item_store computes them.
__device__ __forceinline__ void kitty_codes(const DecodeArgs& a, int64_t blk, int item, int lane,
                                            const u32x4 (&x)[4], const KittyKey& k,
                                            KittyLds& s, int n_boost) {
#pragma clang fp contract(off)
  constexpr int kWpt = kD / 16;              // dense key words per token
  const int c0 = 16 * item, q = lane & 1, hpt = n_boost >> 4;
  const uint32_t m16 = s.bmask[item];
  int base = 0;                              // boosted channels of the items before
  for (int w = 0; w < item; ++w) base += __popc(s.bmask[w]);
  float sc[8], rs[8], mq[8];
  int row[8];
  uint32_t shw[4], mnw[4], bw[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = 8 * q + e;
    const bool boosted = (m16 >> j) & 1u;
    row[e] = boosted ? base + __popc(m16 & ((1u << j) - 1u)) : n_boost;
    mq[e] = boosted ? 15.0f : 3.0f;
    const uint16_t sh = f2h(k.rng[e] / mq[e]);
    const uint16_t l16 = from_order_key(k.lo[e]);
    sc[e] = h2f(sh);
    rs[e] = sc[e] == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sc[e]);   // as group_stat
    if (e & 1) {
      shw[e >> 1] |= (uint32_t)sh << 16;
      mnw[e >> 1] |= (uint32_t)l16 << 16;
    } else {
      shw[e >> 1] = sh;
      mnw[e >> 1] = l16;
    }
    bw[e >> 2] |= (uint32_t)row[e] << (8 * (e & 3));
  }
  if (lane < 2) {
    const int64_t m_off = blk * kD + c0 + 8 * q;
    *reinterpret_cast<u32x4*>(a.c.k_scale + m_off) = u32x4{shw[0], shw[1], shw[2], shw[3]};
    *reinterpret_cast<u32x4*>(a.c.k_min + m_off) = u32x4{mnw[0], mnw[1], mnw[2], mnw[3]};
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(a.c.k_bidx + m_off) = u32x2{bw[0], bw[1]};
  }
  // nibble e of nib[i]: the code of channel c0 + 8q + e at token l/2 + 32i
  uint32_t nib[4];
  bool near = false;
  auto pack = [&](bool exact) {
    float dev = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t acc = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yc = fminf(quot(x[i][e >> 1], e & 1, k.mn[e], sc[e], rs[e], exact), mq[e]);
        acc += round_bits(yc, dev) << (4 * e);
      }
      nib[i] = acc - magic_sum(4, 8);
    }
    if (!exact) near = dev > kTieWindow;
  };
  pack(false);
  if (__any(near)) pack(true);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = (lane >> 1) + 32 * i;
    uint32_t part = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) part |= ((nib[i] >> (4 * e)) & 3u) << (2 * (8 * q + e));
    // the two lanes of a token hold the two halves of one word
    const uint32_t word = part | row_lane<kXor1>(part);
    if (q == 0) a.c.k_codes[(blk * kG + t) * kWpt + item] = word;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (row[e] < n_boost)
        atomicOr(&s.hi[t * hpt + (row[e] >> 4)], ((nib[i] >> (4 * e + 2)) & 3u)
                                                     << (2 * (row[e] & 15)));
  }
}

}  // namespace app
}  // namespace kvq
