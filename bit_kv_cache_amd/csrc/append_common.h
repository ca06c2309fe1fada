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

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int e) {
  return (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
}
__device__ __forceinline__ uint32_t half_key(const u32x4& v, int e) {
  return order_key(half_of(v, e));
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

// Code of x in a group (mn, s, rs) as quant_code_rcp computes it, in two
// parts: quot() is the quotient by the reciprocal, or (exact) by the IEEE
// division, and near() says whether the former lies within quant_code_rcp's
// tie window.  An item first codes every value by the reciprocal and notes
// whether any value of the wave lies within the window; only then does it
// code the item again by the IEEE quotient, so the window costs no branch
// per value (ONE_CHECK; otherwise quant_code_rcp itself, value by value,
// which keeps fewer registers live).  Outside the window both quotients give
// the same code, so the codes are quant_code_rcp's either way.
__device__ __forceinline__ float quot(float x, float mn, float s, float rs, bool exact) {
#pragma clang fp contract(off)
  return exact ? (x - mn) / s : (x - mn) * rs;
}
__device__ __forceinline__ bool near_tie(float y) {
  return __builtin_fabsf((y - __builtin_floorf(y)) - 0.5f) < 0x1p-16f;
}
__device__ __forceinline__ uint32_t code_of(float y, float s, float maxq) {
  return s == 0.0f ? 0u : (uint32_t)__builtin_rintf(fminf(fmaxf(y, 0.0f), maxq));
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
    // per channel over the 128 tokens: the lane's 4, then the 32 lanes with
    // the same q
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = half_key(x[0], e);
      hi[e] = lo[e];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        lo[e] = min(lo[e], half_key(x[i], e));
        hi[e] = max(hi[e], half_key(x[i], e));
      }
    }
    // the 8 lanes of the row with this q (DPP), then the four rows
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = min(lo[e], row_lane<kRor8>(lo[e]));
      hi[e] = max(hi[e], row_lane<kRor8>(hi[e]));
      lo[e] = min(lo[e], row_lane<kRor4>(lo[e]));
      hi[e] = max(hi[e], row_lane<kRor4>(hi[e]));
      lo[e] = min(lo[e], row_lane<kXor2>(lo[e]));
      hi[e] = max(hi[e], row_lane<kXor2>(hi[e]));
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = min(lo[e], (uint32_t)__shfl_xor((int)lo[e], o));
        hi[e] = max(hi[e], (uint32_t)__shfl_xor((int)hi[e], o));
      }
    float mn[8], sc[8], rs[8];
    uint32_t shw[4], mnw[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t l16 = from_order_key(lo[e]);
      const uint16_t sh = group_scale(h2f(l16), h2f(from_order_key(hi[e])), kMaxq);
      mn[e] = h2f(l16);
      sc[e] = h2f(sh);
      rs[e] = __builtin_amdgcn_rcpf(sc[e]);   // within an ulp: enough (quant_code_rcp)
      if (e & 1) {
        shw[e >> 1] |= (uint32_t)sh << 16;
        mnw[e >> 1] |= (uint32_t)l16 << 16;
      } else {
        shw[e >> 1] = sh;
        mnw[e >> 1] = l16;
      }
    }
    if (lane < 2) {
      const int64_t m_off = blk * kD + c0 + 8 * q;
      *reinterpret_cast<u32x4*>(a.c.k_scale + m_off) = u32x4{shw[0], shw[1], shw[2], shw[3]};
      *reinterpret_cast<u32x4*>(a.c.k_min + m_off) = u32x4{mnw[0], mnw[1], mnw[2], mnw[3]};
    }
    // codes of token t: channel c0 + 8q + e at bits BITS (c0 + 8q + e) mod
    // 32 of key word (c0 + 8q + e) / kFpi
    uint32_t parts[4];
    bool near = false;
    auto pack = [&](bool exact) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        parts[i] = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = h2f(half_of(x[i], e));
          uint32_t c;
          if constexpr (ONE_CHECK) {
            const float y = quot(xv, mn[e], sc[e], rs[e], exact);
            if (!exact) near = near || near_tie(y);
            c = code_of(y, sc[e], kMaxq);
          } else {
            c = quant_code_rcp(xv, mn[e], sc[e], rs[e], kMaxq);
          }
          parts[i] |= c << (BITS * ((8 * q + e) % kFpi));
        }
      }
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
    // per token over the 128 channels: the lane's 8, then the 16 lanes with
    // the same r
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = half_key(x[i], 0);
      hi[i] = lo[i];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        lo[i] = min(lo[i], half_key(x[i], e));
        hi[i] = max(hi[i], half_key(x[i], e));
      }
    }
    // the 16 lanes of the row (DPP)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = min(lo[i], row_lane<kRor8>(lo[i]));
      hi[i] = max(hi[i], row_lane<kRor8>(hi[i]));
      lo[i] = min(lo[i], row_lane<kRor4>(lo[i]));
      hi[i] = max(hi[i], row_lane<kRor4>(hi[i]));
      lo[i] = min(lo[i], row_lane<kXor2>(lo[i]));
      hi[i] = max(hi[i], row_lane<kXor2>(hi[i]));
      lo[i] = min(lo[i], row_lane<kXor1>(lo[i]));
      hi[i] = max(hi[i], row_lane<kXor1>(hi[i]));
    }
    float mn[4], sc[4], rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t l16 = from_order_key(lo[i]);
      const uint16_t sh = group_scale(h2f(l16), h2f(from_order_key(hi[i])), kMaxq);
      mn[i] = h2f(l16);
      sc[i] = h2f(sh);
      rs[i] = __builtin_amdgcn_rcpf(sc[i]);
      if (q == 0) {
        const int64_t m_off = blk * kG + t0 + r + 4 * i;
        a.c.v_scale[m_off] = sh;
        a.c.v_min[m_off] = l16;
      }
    }
    // codes: token t0 + j (j = r + 4i) at bits BITS (j mod kFpi) of word row
    // (t0 + j) / kFpi of its channel; the 4 lanes with the same q hold the
    // item's 16 tokens of a channel
    constexpr int kRows = 16 / kFpi;   // word rows of the item (1 or 2)
    uint32_t part[8][kRows];           // this lane's codes of channel 8q + e
    bool near = false;
    auto pack = [&](bool exact) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int w = 0; w < kRows; ++w) part[e][w] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = r + 4 * i;
          const float xv = h2f(half_of(x[i], e));
          uint32_t c;
          if constexpr (ONE_CHECK) {
            const float y = quot(xv, mn[i], sc[i], rs[i], exact);
            if (!exact) near = near || near_tie(y);
            c = code_of(y, sc[i], kMaxq);
          } else {
            c = quant_code_rcp(xv, mn[i], sc[i], rs[i], kMaxq);
          }
          // i is a compile-time index: j / kFpi == (4 i) / kFpi for r < 4
          part[e][(4 * i) / kFpi] |= c << (BITS * (j % kFpi));
        }
      }
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

}  // namespace app
}  // namespace kvq
