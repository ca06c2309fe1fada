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
// Work split: block = 4 waves on one (batch, kv head) and one chunk of groups
// plus a slice of the fp16 sink/residual window (so every block carries the
// same load and the grid runs in one round of resident blocks).  Each wave
// owns whole groups (round robin) with its own online softmax state and
// software-pipelined loads (the next group's keys load during q.K^T's
// successors, its values during p.V's).  At the chunk end the waves and the
// window slice merge in LDS and the block writes its partial (m, l, acc); the
// log-sum-exp merge kernel combines the chunks.

#include <type_traits>

#include "kvq_internal.h"
#include "merge_common.h"
#include "append_common.h"

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

// 2-bit word (codes 0..15 at bits 2i) -> operand quad q (0 or 1).  Element
// pairs (lo half, hi half) j = 0..7 hold codes (j, j+8) at in-half bit
// offset p(j) = {0,2,4,6,8,0,2,4}; quad 0 holds j = 0..3, quad 1 j = 4..7.
__device__ __forceinline__ u32x4 conv2_q(uint32_t w, int q) {
  if (q == 0) return u32x4{w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
  const uint32_t s = w >> 10;
  return u32x4{w & 0x03000300u, s & 0x00030003u, s & 0x000C000Cu, s & 0x00300030u};
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

// DPP lane moves (VALU, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

// max / sum over the 16 lanes of a row (every lane gets the result)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kRowRor8>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  return fmaxf(v, dpp<kQuadXor1>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kRowRor8>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kQuadXor2>(v);
  return v + dpp<kQuadXor1>(v);
}
// value of lane l ^ 32 (gfx950 v_permlane32_swap)
__device__ __forceinline__ float xor32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Streaming loads: every cache byte is read once per step, so the loads are
// non-temporal (no reuse expected in the caches).
template <typename T>
__device__ __forceinline__ T ldnt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

template <int BITS>
struct KeyLoad {
  static constexpr int KW = BITS == 2 ? 2 : 4;   // key words per lane per tile
  uint32_t kw[8][KW];                           // 8 tiles of 16 tokens
  u32x4 kmin[4];                                // key minima, natural order (bias MFMA)
  u32x2 ks[2];                                  // key scales of the A-prep chunk
};

template <int BITS>
struct ValueLoad {
  static constexpr int VR = BITS == 2 ? 2 : 4;   // value word rows per lane group
  u32x4 vw[VR][2];
  u32x2 vs[2], vm[2];                           // value scale / min of the P' chunk
};

// Offset (elements) of the two 4-element runs of an A-prep chunk.
template <int BITS>
__device__ __forceinline__ int run_stride() { return BITS == 2 ? 8 : 4; }

// Per-lane byte offsets of a wave's loads inside one group (uniform bases
// come from the group index; lane offsets stay 32-bit).
template <int BITS>
struct LaneOffsets {
  uint32_t kw;      // key words of tile 0 (tile t adds 16 * t * WPT * 4)
  uint32_t kmeta;   // key scale run 0 inside the group's [D] row
  uint32_t kmin;    // key minima of K-step 0 (natural order) inside that row
  uint32_t vw;      // value words (row VR*kq, channel 4n)
  uint32_t vmeta;   // value scale/min run 0 inside the group's [G] tokens
};

// blk: the group's block (page) in the cache arrays
template <int BITS>
__device__ __forceinline__ void load_keys(const DecodeArgs& a, int64_t blk,
                                          const LaneOffsets<BITS>& o, KeyLoad<BITS>& L) {
  constexpr int WPT = kD / (32 / BITS);
  const char* kb = reinterpret_cast<const char*>(a.c.k_codes) + blk * kG * WPT * 4 + o.kw;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (BITS == 2) {
      const u32x2 v = ldnt<u32x2>(kb + 16 * t * WPT * 4);
      L.kw[t][0] = v[0];
      L.kw[t][1] = v[1];
    } else {
      const u32x4 v = ldnt<u32x4>(kb + 16 * t * WPT * 4);
#pragma unroll
      for (int i = 0; i < KeyLoad<BITS>::KW; ++i) L.kw[t][i] = v[i];
    }
  }
  const char* km = reinterpret_cast<const char*>(a.c.k_min) + blk * kD * 2 + o.kmin;
#pragma unroll
  for (int c = 0; c < 4; ++c) L.kmin[c] = ldnt<u32x4>(km + 64 * c);
  const char* ks = reinterpret_cast<const char*>(a.c.k_scale) + blk * kD * 2 + o.kmeta;
  L.ks[0] = ldnt<u32x2>(ks);
  L.ks[1] = ldnt<u32x2>(ks + 2 * run_stride<BITS>());
}

template <int BITS>
__device__ __forceinline__ void load_values(const DecodeArgs& a, int64_t blk,
                                            const LaneOffsets<BITS>& o, ValueLoad<BITS>& L) {
  constexpr int FPI = 32 / BITS;
  constexpr int VR = ValueLoad<BITS>::VR;
  const char* vb = reinterpret_cast<const char*>(a.c.v_codes) + blk * (kG / FPI) * kD * 4 + o.vw;
#pragma unroll
  for (int i = 0; i < VR; ++i)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      L.vw[i][e] = ldnt<u32x4>(vb + (i * kD + 64 * e) * 4);
  const int64_t t0 = blk * kG * 2;
  const char* vs = reinterpret_cast<const char*>(a.c.v_scale) + t0 + o.vmeta;
  const char* vm = reinterpret_cast<const char*>(a.c.v_min) + t0 + o.vmeta;
  L.vs[0] = ldnt<u32x2>(vs);
  L.vs[1] = ldnt<u32x2>(vs + 2 * run_stride<BITS>());
  L.vm[0] = ldnt<u32x2>(vm);
  L.vm[1] = ldnt<u32x2>(vm + 2 * run_stride<BITS>());
}

// fp16 element e (= 2r + half) of an A-prep chunk from its two 4-element runs
__device__ __forceinline__ float chunk_elem(const u32x2 (&run)[2], int e) {
  const uint32_t w = run[e & 1][(e >> 1) >> 1];
  return h2f((uint16_t)(((e >> 1) & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

template <int GQA>
struct WaveLds {
  static constexpr int ROWS = 2 * GQA;             // A rows: (head, hi/lo)
  // rows padded by one: the A-prep lanes of one write pass differ in c and
  // kq, which would otherwise put their 16-byte writes 512 bytes apart, on
  // the same LDS banks
  static constexpr int RS = ROWS + 1;
  union {
    struct {
      u32x4 ak[4][4][RS];                          // key A operand [c][kq][row]
      u32x4 av[4][4][RS];                          // value A operand [c][kq][row]
    } op;
    uint32_t vt[kD][8];                            // fp16 window tile, transposed:
                                                   // [channel][token pair]
  };
  float p[GQA][kG + 4];                            // probabilities of the group (rows
                                                   // padded: heads 4 banks apart)
  float alpha[GQA];
  f32x4 qhat[GQA / 4][2][64];                      // scaled query of the A-prep lanes
                                                   // (lane-minor: 16-byte lane stride)
};

template <int GQA>
struct MergeLds {
  float num[kWaves][GQA][kD];
  float m[kWaves][GQA], l[kWaves][GQA], mt[kWaves][GQA];
};

template <int GQA>
struct MfmaLds {
  union {
    struct {
      WaveLds<GQA> w[kWaves];
      u32x4 zero;
    } main;
    MergeLds<GQA> merge;
  } u;
  u32x4 bias_a[4][4][16];                          // bias A operand [c][kq][row]
  int bad;                                         // a group's page lies outside the pool
  int last;                                        // last block of its head (in-launch merge)
};

template <int BITS, int GQA>
__global__ __launch_bounds__(kThreadsM, mfma_blocks_per_cu(BITS, GQA)) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int TPC = GQA == 4 ? 2 : 1;  // tiles per QK accumulator (row slots)
  constexpr int NFRAG = 8 / TPC;         // QK accumulators per group
  constexpr int NH = GQA / 4;            // A-prep heads per lane (1 or 2)
  __shared__ MfmaLds<GQA> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kq = lane >> 4;   // operand lane coordinates
  int chunk, head32;
  xcd_part_head(chunk, head32);
  const int64_t head = head32;
  const int64_t b = head / a.H_kv, hk = head % a.H_kv;
  const uint16_t* qrow = a.q + ((b * a.H_q) + hk * GQA) * kD;

  // ---------------------------------------------------------------- first loads
  // The wave's first group is requested before anything else, so its latency
  // overlaps the window slice and the operand set-up below.
  const int64_t gb = (int64_t)chunk * a.groups_per_chunk;
  const int64_t ge = min<int64_t>(seq_groups(a, b, kG), gb + a.groups_per_chunk);
  const int ph = lane >> 4;
  const int pc = lane & 3, pkq = (lane >> 2) & 3;
  LaneOffsets<BITS> lo;
  {
    constexpr int WPT = kD / (32 / BITS);
    lo.kw = (uint32_t)((n * WPT + KeyLoad<BITS>::KW * kq) * 4);
    lo.kmeta = (uint32_t)(chunk_index<BITS>(pc, pkq, 0) * 2);
    lo.vw = (uint32_t)((ValueLoad<BITS>::VR * kq * kD + 4 * n) * 4);
    lo.vmeta = lo.kmeta;
    lo.kmin = (uint32_t)(8 * kq * 2);
  }
  KeyLoad<BITS> kl;
  ValueLoad<BITS> vl;
  // a group's block (page); a page outside the pool reads block 0 and
  // poisons the block's result
  bool bad_page = false;
  auto blk_of = [&](int64_t gg) -> int64_t {
    const int64_t bk = group_block(a.c, head, gg, kG);
    bad_page = bad_page || bk < 0;
    return bk < 0 ? 0 : bk;
  };
  int64_t g = gb + wave;
  if (g < ge) {
    const int64_t blk = blk_of(g);
    load_keys<BITS>(a, blk, lo, kl);
    load_values<BITS>(a, blk, lo, vl);
  }

  // ---------------------------------------------------------------- quantized groups
  WaveLds<GQA>& L = sh.u.main.w[wave];
  if (tid == 0) {
    sh.u.main.zero = u32x4{0u, 0u, 0u, 0u};
    sh.bad = 0;
  }

  // this lane's A-prep heads (ph, ph + 4) and chunk (pc, pkq)
  // q * sm * log2e * 2^(24 - offset) of this lane's A-prep elements, in LDS
  float qmax = 0.f, qmax_n = 0.f;
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    float qh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = chunk_index<BITS>(pc, pkq, e);
      const float qv = h2f(qrow[(ph + 4 * j) * kD + ch]) * a.qscale;
      qh[e] = qv * exp2i(24 - code_offset<BITS>(ch));
      qmax = fmaxf(qmax, fabsf(qh[e]));
      qmax_n = fmaxf(qmax_n, fabsf(qv));
    }
    L.qhat[j][0][lane] = f32x4{qh[0], qh[1], qh[2], qh[3]};
    L.qhat[j][1][lane] = f32x4{qh[4], qh[5], qh[6], qh[7]};
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    qmax = fmaxf(qmax, __shfl_xor(qmax, o));
    qmax_n = fmaxf(qmax_n, __shfl_xor(qmax_n, o));
  }
  const int e_q = ceil_exp(qmax);
  // The bias / window operand below is q*sm*log2e times 2^(8 - e_n), its
  // largest entry below 2^8, so that small entries stay normal fp16 numbers
  // in the hi/lo split; products from it are scaled back by 2^(e_n - 8).
  const int e_n = ceil_exp(qmax_n);
  const float q_nat_unscale = exp2i(max(-126, min(127, e_n - 8)));

  // bias operand: hi/lo of q*sm*log2e in natural channel order, rows (head,
  // hi/lo); built once per block in LDS (wave w builds K-step w)
  {
    const int m = lane & 15, c = wave;
    const int h = (m % (2 * GQA)) >> 1, hl = m & 1;
    const float qs = a.qscale * exp2i(max(-126, min(127, 8 - e_n)));
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = h2f(qrow[h * kD + 32 * c + 8 * kq + e]) * qs;
    u32x4 hi, lo;
    split_hilo(v, hi, lo);
    sh.bias_a[c][kq][m] = hl ? lo : hi;
  }

  // per-wave online softmax state: this lane's QK heads hA, hA + 1
  const int rq = lane >> 4;
  const int hA = GQA == 4 ? 2 * (rq & 1) : 2 * rq;
  const bool pv_rows = GQA == 8 || rq < 2;  // lanes holding real p.V rows
  float m_run[2] = {kNegInfM, kNegInfM};
  float l_part[2] = {0.f, 0.f};
  float mterm[NH];                          // sum_t p_t * value min, A-prep heads
#pragma unroll
  for (int j = 0; j < NH; ++j) mterm[j] = 0.f;
  int e_v = -1000;                          // running value-side exponent
  f32x4 acc[8];                             // p.V accumulators, 8 channel blocks
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int m_row = lane & 15;
  // LDS address of this lane's A operand chunk (K-step 0), per row slot; lanes
  // whose rows are unused in a slot read the zero block instead
  const u32x4* ak_ptr[TPC];
  int ak_step[TPC];                         // K-step stride (0 on the zero block)
#pragma unroll
  for (int slot = 0; slot < TPC; ++slot) {
    const bool mine = TPC == 1 || (m_row >> 3) == slot;
    ak_ptr[slot] = mine ? &L.op.ak[0][kq][TPC == 1 ? m_row : (m_row & 7)] : &sh.u.main.zero;
    ak_step[slot] = mine ? 4 * WaveLds<GQA>::RS : 0;
  }
  const bool av_mine = m_row < 2 * GQA;
  const u32x4* av_ptr = av_mine ? &L.op.av[0][kq][m_row] : &sh.u.main.zero;
  const int av_step = av_mine ? 4 * WaveLds<GQA>::RS : 0;
  __syncthreads();

  // One group of this wave.  With PREFETCH the next group's keys are fetched
  // right after q.K^T and its values right after p.V (unconditionally, so the
  // wait counters stay exact); the wave's last group runs without.
  auto group_step = [&](int64_t g, auto prefetch_tag) {
    constexpr bool PREFETCH = decltype(prefetch_tag)::value;
    const int64_t gn = g + kWaves;

    // ---- key A operand: (q s) 2^(24-offset) 2^-E_K as hi/lo rows, via LDS
    float ks[8];
    float smax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ks[e] = chunk_elem(kl.ks, e);
      smax = fmaxf(smax, ks[e]);
    }
    smax = row_max16(smax);
    const int e_k = e_q + ceil_exp(smax) - 15;
    const float sk = exp2i(max(-126, min(127, -e_k)));
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const f32x4 q0 = L.qhat[j][0][lane], q1 = L.qhat[j][1][lane];
      const float qh[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = qh[e] * ks[e] * sk;
      u32x4 hi, lo;
      split_hilo(v, hi, lo);
      const int h = ph + 4 * j;
      L.op.ak[pc][pkq][2 * h] = hi;
      L.op.ak[pc][pkq][2 * h + 1] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- bias: sum_d q_d mn_d per head (key minima in natural channel order)
    f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) cb = mfma(sh.bias_a[c][kq][m_row], kl.kmin[c], cb);
    const float biasA = (cb[0] + cb[1]) * q_nat_unscale, biasB = (cb[2] + cb[3]) * q_nat_unscale;

    // ---- q.K^T
    const float ek = exp2i(max(-126, min(127, e_k)));
    float logit[NFRAG][2];
    {
      f32x4 cq[NFRAG];
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) cq[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int slot = 0; slot < TPC; ++slot) {
          const u32x4 aq = *(ak_ptr[slot] + c * ak_step[slot]);
#pragma unroll
          for (int f = 0; f < NFRAG; ++f) {
            const int t = f * TPC + slot;
            const u32x4 bq = BITS == 2 ? conv2_q(kl.kw[t][c >> 1], c & 1) : conv4(kl.kw[t][c]);
            cq[f] = mfma(aq, bq, cq[f]);
          }
        }
      }
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        logit[f][0] = fmaf(cq[f][0] + cq[f][1], ek, biasA);
        logit[f][1] = fmaf(cq[f][2] + cq[f][3], ek, biasB);
      }
    }
    // the key registers are free: fetch the next group's keys
    const int64_t blk_n = PREFETCH ? blk_of(gn) : 0;
    if (PREFETCH) load_keys<BITS>(a, blk_n, lo, kl);

    // ---- online softmax over the group (per head, this wave)
    float alpha[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = logit[0][j];
#pragma unroll
      for (int f = 1; f < NFRAG; ++f) v = fmaxf(v, logit[f][j]);
      v = row_max16(v);
      if (GQA == 4) v = fmaxf(v, xor32(v));
      const float m_new = fmaxf(m_run[j], v);
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
    if (n == 0 && pv_rows) {
      L.alpha[hA] = alpha[0];
      L.alpha[hA + 1] = alpha[1];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value A operand: p s_t 2^(24-offset) 2^-E_V as hi/lo rows, via LDS
    float vs[8];
    float vmax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vs[e] = chunk_elem(vl.vs, e);
      vmax = fmaxf(vmax, vs[e]);
    }
    vmax = row_max16(vmax);
    const int e_v_new = max(e_v, ceil_exp(vmax) + 9);
    const float vshift = exp2i(max(-126, min(127, e_v - e_v_new)));
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
        mt = fmaf(p, chunk_elem(vl.vm, e), mt);
      }
      mterm[j] = fmaf(mterm[j], al, mt);
      u32x4 hi, lo;
      split_hilo(v, hi, lo);
      L.op.av[pc][pkq][2 * h] = hi;
      L.op.av[pc][pkq][2 * h + 1] = lo;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- rescale the p.V accumulators (alpha and the exponent change)
    {
      const float f0 = pv_rows ? L.alpha[2 * rq] * vshift : 0.f;
      const float f1 = pv_rows ? L.alpha[2 * rq + 1] * vshift : 0.f;
      if (!__all((f0 == 1.f && f1 == 1.f) || !pv_rows)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[i][0] *= f0;
          acc[i][1] *= f0;
          acc[i][2] *= f1;
          acc[i][3] *= f1;
        }
      }
    }

    // ---- p.V
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 apv = *(av_ptr + c * av_step);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int e = blk >> 2, comp = blk & 3;
        const u32x4 bv = BITS == 2 ? conv2_q(vl.vw[c >> 1][e][comp], c & 1) : conv4(vl.vw[c][e][comp]);
        acc[blk] = mfma(apv, bv, acc[blk]);
      }
    }
    // the value registers are free: fetch the next group's values
    if (PREFETCH) load_values<BITS>(a, blk_n, lo, vl);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (g < ge) {
    for (; g + kWaves < ge; g += kWaves) group_step(g, std::true_type{});
    group_step(g, std::false_type{});
  }

  // ---------------------------------------------------------------- fp16 window
  // Window tokens [u0, u1) of sink | residual belong to this block (every
  // block takes an equal slice).  Wave w takes 16-token tiles w, w + 4, ...:
  // q.K^T on the matrix core with the raw fp16 keys as B (natural channel
  // order, the bias operand as A), the same online softmax, and p.V through an
  // LDS transpose of the fp16 values into a natural-scale accumulator.
  f32x4 wacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const int n_win = a.n_sink + seq_res(a, b);
    const int wpc = (n_win + a.n_chunks - 1) / a.n_chunks;
    const int u0 = min(n_win, chunk * wpc), u1 = min(n_win, u0 + wpc);
    auto row = [&](const uint16_t* sink, const uint16_t* res, int u) -> const uint16_t* {
      return u < a.n_sink ? sink + (head * a.sink_cap + u) * kD
                          : res + (head * a.res_cap + (u - a.n_sink)) * kD;
    };
    for (int u = u0 + 16 * wave; u < u1; u += 16 * kWaves) {
      const int nt = min(16, u1 - u);
      // keys of token n (rows past the tile end repeat its last token)
      const uint16_t* kr = row(a.k_sink, a.k_res, u + min(n, nt - 1));
      u32x4 kv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kv[c] = *reinterpret_cast<const u32x4*>(kr + 32 * c + 8 * kq);
      // values: lane (token pair j, 16-channel group cg) -> vt[channel][j]
      {
        const int j = lane & 7, cg = lane >> 3;
        const uint16_t* r0 = row(a.v_sink, a.v_res, u + min(2 * j, nt - 1)) + 16 * cg;
        const uint16_t* r1 = row(a.v_sink, a.v_res, u + min(2 * j + 1, nt - 1)) + 16 * cg;
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(r0);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(r0 + 8);
        const u32x4 y0 = *reinterpret_cast<const u32x4*>(r1);
        const u32x4 y1 = *reinterpret_cast<const u32x4*>(r1 + 8);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t x = q < 4 ? x0[q] : x1[q - 4];
          const uint32_t y = q < 4 ? y0[q] : y1[q - 4];
          L.vt[16 * cg + 2 * q][j] = __builtin_amdgcn_perm(y, x, 0x05040100u);
          L.vt[16 * cg + 2 * q + 1][j] = __builtin_amdgcn_perm(y, x, 0x07060302u);
        }
      }
      f32x4 cw = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) cw = mfma(sh.bias_a[c][kq][m_row], kv[c], cw);
      // rows 8..15 repeat rows 0..7 when GQA == 4
      const bool valid = n < nt && (GQA == 8 || rq < 2);
      float alpha[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float lg = valid ? (cw[2 * j] + cw[2 * j + 1]) * q_nat_unscale : kNegInfM;
        float v = row_max16(lg);
        if (GQA == 4) v = fmaxf(v, xor32(v));
        const float m_new = fmaxf(m_run[j], v);   // finite: the tile has a valid token
        alpha[j] = exp2f(m_run[j] - m_new);
        m_run[j] = m_new;
        const float p = valid ? exp2f(lg - m_new) : 0.f;
        if (GQA == 8 || rq < 2) L.p[hA + j][n] = p;
        l_part[j] = fmaf(l_part[j], alpha[j], p);
      }
      if (n == 0 && pv_rows) {
        L.alpha[hA] = alpha[0];
        L.alpha[hA + 1] = alpha[1];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < NH; ++j) mterm[j] *= L.alpha[ph + 4 * j];
      {
        const float f0 = pv_rows ? L.alpha[2 * rq] : 0.f;
        const float f1 = pv_rows ? L.alpha[2 * rq + 1] : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[i][0] *= f0;
          acc[i][1] *= f0;
          acc[i][2] *= f1;
          acc[i][3] *= f1;
          wacc[i][0] *= f0;
          wacc[i][1] *= f0;
          wacc[i][2] *= f1;
          wacc[i][3] *= f1;
        }
      }
      // A = p (hi/lo rows), tokens 8kq..8kq+7 of the tile (kq < 2)
      u32x4 apw = u32x4{0u, 0u, 0u, 0u};
      if (m_row < 2 * GQA && kq < 2) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = L.p[m_row >> 1][8 * kq + e];
        u32x4 hi, lo;
        split_hilo(v, hi, lo);
        apw = (m_row & 1) ? lo : hi;
      }
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int d = 64 * (blk >> 2) + 4 * n + (blk & 3);
        const u32x4 bv = kq < 2 ? *reinterpret_cast<const u32x4*>(&L.vt[d][4 * kq])
                                : u32x4{0u, 0u, 0u, 0u};
        wacc[blk] = mfma(apw, bv, wacc[blk]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // ---------------------------------------------------------------- block merge
  float lsum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float v = row_sum16(l_part[j]);
    if (GQA == 4) v += xor32(v);
    lsum[j] = v;
  }
  float mtsum[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    mtsum[j] = row_sum16(mterm[j]);
  }
  if (bad_page) sh.bad = 1;
  __syncthreads();   // the per-wave buffers are reused for the merge below
  MergeLds<GQA>& M = sh.u.merge;
  if (n == 0 && pv_rows) {
    M.m[wave][hA] = m_run[0];
    M.m[wave][hA + 1] = m_run[1];
    M.l[wave][hA] = lsum[0];
    M.l[wave][hA + 1] = lsum[1];
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < NH; ++j) M.mt[wave][ph + 4 * j] = mtsum[j];
  }
  __syncthreads();
  if (pv_rows) {
    const int h0 = 2 * rq;
    const float ev = exp2i(max(-126, min(127, e_v)));
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int d = 64 * (blk >> 2) + 4 * n + (blk & 3);
      M.num[wave][h0][d] = fmaf(acc[blk][0] + acc[blk][1], ev, M.mt[wave][h0]) +
                           (wacc[blk][0] + wacc[blk][1]);
      M.num[wave][h0 + 1][d] = fmaf(acc[blk][2] + acc[blk][3], ev, M.mt[wave][h0 + 1]) +
                               (wacc[blk][2] + wacc[blk][3]);
    }
  }
  __syncthreads();
  if (tid == 0 && sh.bad) status_add(a.status, kStatusBadPage);
  for (int i = tid; i < GQA * kD; i += kThreadsM) {
    const int h = i / kD, d = i % kD;
    // every wave's record read up front; empty ones (l = 0) are skipped by
    // selects, not branches, so the reads overlap
    float mw[kWaves], lw[kWaves], nw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = M.m[w][h];
      lw[w] = M.l[w][h];
      nw[w] = M.num[w][h][d];
    }
    float mm = kNegInfM;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = lw[w] > 0.f ? fmaxf(mm, mw[w]) : mm;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(mw[w] - mm);
      num = lw[w] > 0.f ? fmaf(nw[w], f, num) : num;
      den = lw[w] > 0.f ? fmaf(lw[w], f, den) : den;
    }
    if (sh.bad) {   // poisoned: l = 1 keeps the part in the merge, acc NaN
      num = __builtin_nanf("");
      den = 1.f;
      mm = 0.f;
    }
    store_record(a, (b * a.H_q) + hk * GQA + h, chunk, d, mm, den, num);
  }
  if (a.counters) merge_in_launch<GQA>(a, b, hk, head32, sh.last);
  // With DecodeArgs::append the blocks of a head then quantize the group
  // that has filled the residual window: its 16 items (append_common.h), item
  // slot chunk * 4 + wave and every n_chunks * 4-th after it, with no
  // barrier.  At the end of the block they no longer delay its first loads,
  // and the head's blocks share one XCD, so the items' stores into the same
  // cache lines meet in one L2.  (Requesting their inputs before the block
  // merge instead measured slower.)
  if (a.append)
    app::run_items<BITS, 4, true>(a, head, chunk * (kThreadsM / 64) + wave,
                                  a.n_chunks * (kThreadsM / 64), lane);
}

}  // namespace

hipError_t launch_decode_mfma(int bits, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.n_chunks, (unsigned)(a.B * a.H_kv));
  if (bits == 2) {
    return launch_decode_f8f4(a, st);   // fp8 x fp4 matrix cores
  } else {
    if (a.gqa == 4) decode_mfma_kernel<4, 4><<<grid, kThreadsM, 0, st>>>(a);
    else decode_mfma_kernel<4, 8><<<grid, kThreadsM, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvq
