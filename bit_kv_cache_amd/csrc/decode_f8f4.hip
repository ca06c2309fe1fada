// Split-K decode attention for 2-bit codes on gfx950 matrix cores, GQA query
// groups of 4 or 8 heads, group size 128, head dim 128.
//
// The query heads that share a kv head form a dense contraction with the kv
// tile (BitDecoding page, section V.A), so q.K^T and p.V run on
// v_mfma_scale_f32_16x16x128_f8f6f4 with
//
//  * B = the packed 2-bit codes as fp4 (e2m1).  A code c in the low two bits
//    of a nibble whose high bits are clear is the fp4 value c/2, so one AND
//    with 0x33333333 turns a 32-bit word of 16 codes into 8 operand nibbles
//    (the even codes) and a shift plus AND gives the odd ones.  Keys are
//    packed along channels and values along tokens, the contraction axes, so
//    a lane's two words are its 32 contraction elements with no shuffle.
//  * A = the dequantization scales folded into the query / the probabilities
//    (KIVI page Step 4, x = code*scale + min spread over the dot product):
//        q.k_t = sum_d (q_d s_d) code_td + sum_d q_d mn_d
//        p.v_d = sum_t (p_t s_t) code_td + sum_t p_t mn_t
//    Each A value is written as four fp8 (e4m3) digits in four A rows of the
//    same head, so one MFMA per 16 tokens (or 16 channels) serves four heads
//    and the output rows of a head are summed afterwards.  Key side: q_d s_d,
//    scaled by a power of two per group to below 2^8, digit k the
//    round-to-nearest fp8 value of the remaining residual over 2^-4k (about
//    four significant bits each, 16 in all, relative to each value; the
//    MFMA's per-row E8M0 scale undoes the 2^-4k).  Value side: p_t s_t >= 0
//    as a 16-bit fixed-point number relative to its 32-token block's largest,
//    digit k its k-th nibble from the top (fp8 bytes 0..15 are exactly
//    b 2^-9, so no conversion), the block's power of two in the per-row,
//    per-block E8M0 scale.
//  * sum_d q_d mn_d is a vector-ALU dot product in the A-prep lanes; sum_t
//    p_t mn_t is a per-head scalar kept beside the accumulator.
//
// Lane roles (n = lane & 15, r = lane >> 4): lane (n, r) prepares A values of
// head r (and r + 4) for channels / tokens 8n..8n+7, and holds the logits of
// the same head for tokens 16t + n (column n of tile t, so each key load
// instruction reads 512 contiguous bytes); the probabilities pass through a
// small LDS transpose to the lanes that prepare the p.V operand.
// Matrix-core outputs land in lane (n, r) as the four digit rows of head r.
//
// Kitty boost (Kitty page, 3.2 and 4.2): a boosted key channel's code is
// lo + 4 hi; the dense words carry lo, so the high bits add 4 sum_j a_j hi_j
// over the 16 boosted rows, one more scaled product per 16-token tile whose
// B operand is the token's high-bits word and whose A operand gathers the
// boosted channels' digit bytes.
//
// Work split: block = 8 waves on one (batch, kv head) and one chunk of
// groups, one block per CU.  Wave 0 is the loader: it copies each group's
// record (key words, value words, scales and mins, Kitty high bits and
// boosted rows) straight from HBM into an LDS ring with asynchronous
// global-to-LDS loads, several groups in flight, and publishes a slot once
// its data has landed.  Waves 1..7 consume: each claims the next group with
// an LDS counter, copies the operands out of the slot (freeing it) and runs
// both products with its own online softmax.  The block's equal slice of
// the fp16 sink/residual window runs first, as 16-token fp16 tiles.  The
// waves merge in LDS and the block writes its partial (m, l, acc).

#include "kvq_internal.h"
#include "append_common.h"
#include "merge_common.h"
#include "quant_common.h"

#include <type_traits>

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kG = 128;          // tokens per group
// One block per CU: 8 waves (two per SIMD), the first the loader, the
// others consumers; with one chunk per consumer wave (PW), 9 waves: the
// loader and 8 consumers, two per SIMD.
template <int GQA, bool KITTY, bool PW = false>
constexpr int block_waves() { return PW ? 9 : 8; }
constexpr uint32_t kNib = 0x33333333u;
constexpr float kNegInfF = -__builtin_inff();
constexpr int kDigits = 4;        // fp8 digits of an A value
constexpr float kFixMax = 65535.f; // value-side fixed point: M = round(x 65535 / 2^eb) <= 65535
constexpr float kLazyMax = 8.f;    // log2 of the largest probability a group may carry

// ------------------------------------------------------------------ helpers

// A: fp8 e4m3 (format 0) with E8M0 row scale `sa` (the same in every lane of
// a row), B: fp4 e2m1 (format 4) with unit scale (127)
__device__ __forceinline__ f32x4 mfma_f8f4(const v8i& a, const v8i& b, f32x4 c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
}

// The same product with B's per-lane E8M0 block scale sb (the low byte of
// the operand): an MXFP4 block's scale factor, as stored in the cache.
__device__ __forceinline__ f32x4 mfma_f8f4_mx(const v8i& a, const v8i& b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ f32x4 mfma_f16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// fp4 B operand from the two words holding contraction elements 32r..32r+15
// (w0) and 32r+16..32r+31 (w1): nibble j of the operand is element
// 16*(j/16) + 2*(j%8) + (j/8)%2 of the lane's 32.
__device__ __forceinline__ v8i fp4_operand(uint32_t w0, uint32_t w1) {
  return v8i{(int)(w0 & kNib), (int)((w0 >> 2) & kNib), (int)(w1 & kNib),
             (int)((w1 >> 2) & kNib), 0, 0, 0, 0};
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

__device__ __forceinline__ float exp2i(int e) {  // 2^e for e in [-126, 127]
  return __builtin_bit_cast(float, (uint32_t)(max(-126, min(127, e)) + 127) << 23);
}

// smallest e with x < 2^e for finite x >= 0 (x == 0 -> -126)
__device__ __forceinline__ int ceil_exp(float x) {
  const int b = (int)((__builtin_bit_cast(uint32_t, x) >> 23) & 0xFF);
  return b == 0 ? -126 : b - 126;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                              0xF, true));
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero,
// which softmax weights can afford)
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

// max / sum over the 16 lanes of a row (every lane of the row gets it)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kRowRor8>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  return fmaxf(v, dpp<kQuadXor1>(v));
}
__device__ __forceinline__ uint32_t row_max16u(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kRowRor8, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kRowRor4, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, true));
  return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, true));
}

// Largest of 8 non-negative fp16 values (as bits: their order as unsigned
// integers is their numeric order), over the 16 lanes of the row, returned
// as the smallest e with every value < 2^e (-14 for subnormal or zero).
__device__ __forceinline__ int row_exp_f16(const u32x4& v) {
  const uint32_t lo = max(max(v[0] & 0xFFFFu, v[1] & 0xFFFFu), max(v[2] & 0xFFFFu, v[3] & 0xFFFFu));
  const uint32_t hi = max(max(v[0] >> 16, v[1] >> 16), max(v[2] >> 16, v[3] >> 16));
  const uint32_t top = row_max16u(max(lo, hi));
  const int ef = (int)(top >> 10);                 // biased fp16 exponent
  return (ef == 0 ? 1 : ef) - 14;
}

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kRowRor8>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kQuadXor2>(v);
  return v + dpp<kQuadXor1>(v);
}

// Four fp8 digits of four values (x0..x3 -> bytes 0..3 of each digit word).
// Digit k is the nearest fp8 value of what digits 0..k-1 left over, divided
// by 2^(eb - 4k) (a scaled conversion), so each digit adds about four
// significant bits and no residual sinks into the fp8 subnormal range; the
// matrix-core row of digit k carries the block scale 2^-4k, so the rows of a
// value add up to x / 2^eb.
__device__ __forceinline__ void fp8_digits(float x0, float x1, float x2, float x3, int eb,
                                           uint32_t (&d)[kDigits]) {
  typedef short v2s __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    const float sc = exp2i(eb - 4 * k);
    v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x0, x1, sc, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x2, x3, sc, true);
    const int wi = __builtin_bit_cast(int, w);
    d[k] = (uint32_t)wi;
    if (k < kDigits - 1) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wi, sc, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wi, sc, true);
      x0 -= lo[0];
      x1 -= lo[1];
      x2 -= hi[0];
      x3 -= hi[1];
    }
  }
}

// Byte offset, inside row 0 of an A-operand tile (4 lane groups x 32 B), of
// the four even-numbered elements of octet o (items 8o, 8o+2, 8o+4, 8o+6);
// the odd ones sit 8 bytes further.  The B operand's element
// order (fp4_operand) and the f8f6f4 instruction's A byte order fix it: A
// byte i of lane group g is contraction element 16g + (i%16) + 64(i/16).
__device__ __forceinline__ uint32_t a_offset(int o) {
  const int g = o >> 2, w = (o >> 1) & 1;
  const int ga = 2 * (g & 1) + w;
  const int i0 = 16 * (g >> 1) + 4 * (o & 1);
  return (uint32_t)(ga * 32 + i0);
}

// A-operand tile: 16 rows of 4 lane groups x 32 bytes, rows padded to 144
// bytes so the 16 rows a 128-bit read touches fall in different LDS banks.
constexpr int kRowBytes = 144;
typedef uint8_t ATile[16][kRowBytes];

// ------------------------------------------------------------------ LDS

template <int GQA, bool MX>
struct WaveLdsF {
  static constexpr int NH = GQA / 4;
  struct OpTiles {
    ATile ak[NH];                                 // q.K^T A operand [half][row][g*32 + byte]
    ATile av[NH];                                 // p.V A operand
  };
  // MXFP4: the q.K^T operand is built once per block, before the first p.V
  // one, so the two tiles share their bytes
  union OpShared {
    ATile ak[NH];
    ATile av[NH];
  };
  union {
    std::conditional_t<MX, OpShared, OpTiles> op;
    uint32_t vt[kD][10];                          // fp16 window tile, [channel][token pair]
                                                  // (rows padded to 40 bytes)
  };
  float p[GQA][16];                               // window-tile probabilities
  // group probabilities [head][token] (rows padded: 4 heads, 4 banks apart);
  // the MXFP4 path keeps them in registers
  float pt[MX ? 1 : GQA][MX ? 1 : kG + 4];
};

template <int GQA, int NW>
struct MergeLdsF {
  float num[NW][GQA][kD];
  float m[NW][GQA], l[NW][GQA];
};

// Ring of group records filled by the loader wave: slot layout (bytes)
//   [0, 4096)      key words of the 128 tokens in 16-token tiles of 512 B,
//                  each the first 16-B halves of its tokens, then the second
//   [4096, 8192)   value words, 8 rows of 128 channels, as in the cache
//   [8192, 8448)   key scale of the 128 channels (fp16), then key min,
//   [8704, 8960)   value scale of the 128 tokens, then value min
// and with the Kitty boost (16 boosted key channels per group)
//   [9216, 9728)   high-bits word of each token (boosted rows 0..15)
//   [9728, 9856)   boosted row of each channel (16 = not boosted), then pad
constexpr int kSlotV = 4096, kSlotKs = 8192, kSlotKm = 8448, kSlotVs = 8704, kSlotVm = 8960;
constexpr int kSlotHi = 9216, kSlotBidx = 9728;
//
// MXFP4 cache (128 tokens of a head per group):
//   [0, 8192)      key codes of the 128 tokens, 64 bytes each; row 16 i + k
//                  holds token 8 k + i (the q.K^T tiles' column order)
//   [8192, 16384)  value codes, 16 rows of 8 tokens x 128 channels, as in the cache
//   [16384, 16896) key E8M0 scales of the 128 tokens (4 blocks of 32 channels each)
//   [16896, 17408) value E8M0 scales, 4 rows (32-token blocks) of 128 channels
constexpr int kMxV = 8192, kMxKs = 16384, kMxVs = 16896;
template <bool KITTY, bool MX>
constexpr int slot_bytes() { return MX ? 17408 : KITTY ? 10240 : 9216; }
template <bool KITTY, bool MX>
constexpr int dma_per_group() { return MX ? 17 : KITTY ? 10 : 9; }
template <int GQA, bool KITTY, bool MX, bool PW = false>
constexpr int ring_slots() {
  return PW ? 8 : MX ? (GQA == 4 ? 6 : 5) : GQA == 4 ? (KITTY ? 10 : 12) : 6;
}
// groups the loader keeps in flight: fewer than ring_slots, (DF - 1) groups
// of copies (plus each group's flag copy) within the vector-memory counter's
// 63, and for plain codes fewer still, as measured: 4 with one chunk per
// block (the 32K step 0.75 us faster than with 7) and 3 with one chunk per
// consumer wave (the 1M-token step 5 us faster than with 7; 2 is 10 us
// slower).
template <int GQA, bool KITTY, bool MX, bool PW = false>
constexpr int in_flight() {
  constexpr int per = dma_per_group<KITTY, MX>() + 1;
  constexpr int rs = ring_slots<GQA, KITTY, MX, PW>();
  constexpr int cap = rs - 1 < 63 / per + 1 ? rs - 1 : 63 / per + 1;
  constexpr int want = PW ? 3 : (KITTY || MX) ? cap : 4;
  return want < cap ? want : cap;
}

template <int GQA, bool KITTY, bool MX, bool PW = false>
struct LdsF {
  static constexpr int R = ring_slots<GQA, KITTY, MX, PW>();
  static constexpr int NW = block_waves<GQA, KITTY, PW>();
  union {
    WaveLdsF<GQA, MX> w[NW - 1];
    MergeLdsF<GQA, NW> merge;
    app::KittyLds kitty;      // the Kitty append's key items, after the merge
  } u;
  alignas(16) uint8_t ring[R][slot_bytes<KITTY, MX>()];
  int ready[R];     // chunk-relative group (mod kSeqLen) a slot holds once its data has arrived
  int empty[R];     // the group a slot may receive next (its previous one was copied out)
  int next_group;   // next group a consumer claims
  int stalled;      // bit 0: a wait ran past its spin limit; bit 1: a page outside the pool
  int last;         // this block is the last of its head to finish (in-launch merge)
};

struct Operands {
  uint32_t kw[8][2];     // key words: tile t, token 16t + n, words 2r, 2r + 1
  uint32_t hw[8];        // Kitty: high-bits word of token 16t + n
  u32x4 ks, kmin;        // key scale / min of channels 8n..8n+7
  u32x4 vw[2][2];        // value words: rows 2r, 2r + 1; channels 4n.. and 64 + 4n..
  u32x4 vs, vmn;         // value scale / min of tokens 8n..8n+7
};

// One 1 KB wave-wide copy from global memory into LDS: lane i's 16 bytes at
// gptr land at LDS byte address lds + 16 i.  Written as an instruction
// rather than the compiler builtin because the compiler makes every later
// LDS access wait for all such copies in flight, which would serialize the
// loader; the loader waits for its copies itself (loader_wait).  The cache
// is read once per step: the copies are marked non-temporal (streaming).
__device__ __forceinline__ void dma_1k(uint32_t lds, const void* gptr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr),
               "s"(lds)
               : "memory");
}

// One 4-byte copy from global memory into LDS byte address lds (issued by
// one lane): the ready flag of a ring slot.
__device__ __forceinline__ void dma_flag(uint32_t lds, const void* gptr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(lds)
               : "memory");
}

// Sequence table 0, 1, ..., kSeqLen - 1 in global memory: the values the
// ring's ready flags are copied from.
constexpr int kSeqLen = 4096;
struct SeqTable {
  int v[kSeqLen];
  constexpr SeqTable() : v() {
    for (int i = 0; i < kSeqLen; ++i) v[i] = i;
  }
};
__device__ constexpr SeqTable kSeq{};

// Wait until at most N of this wave's vector-memory loads are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T lds_load(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <typename T>
__device__ __forceinline__ void lds_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Spin (with sleeps) until *p == want; false if the spin limit ran out (the
// caller then stops, so every wave always reaches the end of the kernel).
// The flag is compared as a wave-uniform (scalar) value: a per-lane compare
// would let the compiler treat the loop exit as divergent and restructure
// the caller's loop so that lanes run different iterations.
constexpr uint32_t kSpinLimit = 1u << 20;
__device__ __forceinline__ bool spin_until(const int* p, int want) {
  for (uint32_t i = 0; i < kSpinLimit; ++i) {
    if (__builtin_amdgcn_readfirstlane(lds_load(p)) == want) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (the hardware executes one wave's LDS operations in order; this keeps
// the compiler from moving the accesses across each other, while other
// instructions may still be scheduled across it).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 8 fp16 of a u32x4 as floats
__device__ __forceinline__ void unpack8(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f_lo(v[i]);
    x[2 * i + 1] = h2f_hi(v[i]);
  }
}

// Digits of 8 values (items 8o..8o+7) over 2^eb into rows 4*hr..4*hr+3 of an
// A tile.
__device__ __forceinline__ void write_digits(ATile& tile, int hr, uint32_t off,
                                             const float (&x)[8], int eb) {
  uint32_t de[kDigits], dodd[kDigits];
  fp8_digits(x[0], x[2], x[4], x[6], eb, de);
  fp8_digits(x[1], x[3], x[5], x[7], eb, dodd);
  uint8_t* base = &tile[4 * hr][0] + off;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes) = de[k];
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes + 8) = dodd[k];
  }
}

// Fixed-point digits of four non-negative values (x0..x3 -> bytes 0..3 of each
// digit word): M = round(x S) with x S < 65535.5 (an integer in the low
// mantissa bits of x S + 2^23), and digit k is nibble 3 - k of M as an fp8
// byte.  The e4m3 bytes 0..15 are the values b 2^-9 (subnormals, then the
// first binade), so a nibble is its own fp8 encoding and no conversion is
// needed; the matrix-core row of digit k carries 2^(12 - 4k) in its scale.
__device__ __forceinline__ void fixed_digits(float x0, float x1, float x2, float x3, float S,
                                             uint32_t (&d)[kDigits]) {
  constexpr float kRound = 8388608.f;   // 2^23
  const uint32_t u0 = __builtin_bit_cast(uint32_t, fmaf(x0, S, kRound));
  const uint32_t u1 = __builtin_bit_cast(uint32_t, fmaf(x1, S, kRound));
  const uint32_t u2 = __builtin_bit_cast(uint32_t, fmaf(x2, S, kRound));
  const uint32_t u3 = __builtin_bit_cast(uint32_t, fmaf(x3, S, kRound));
  // the four 16-bit M side by side, then their nibbles spread into bytes
  const uint32_t p01 = __builtin_amdgcn_perm(u1, u0, 0x05040100u);
  const uint32_t p23 = __builtin_amdgcn_perm(u3, u2, 0x05040100u);
  const uint32_t lo01 = p01 & 0x0F0F0F0Fu, hi01 = (p01 >> 4) & 0x0F0F0F0Fu;
  const uint32_t lo23 = p23 & 0x0F0F0F0Fu, hi23 = (p23 >> 4) & 0x0F0F0F0Fu;
  d[0] = __builtin_amdgcn_perm(hi23, hi01, 0x07050301u);   // bits 12..15 of each M
  d[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07050301u);   // bits 8..11
  d[2] = __builtin_amdgcn_perm(hi23, hi01, 0x06040200u);   // bits 4..7
  d[3] = __builtin_amdgcn_perm(lo23, lo01, 0x06040200u);   // bits 0..3
}

// Fixed-point digits of 8 non-negative values (items 8o..8o+7) into rows
// 4*hr..4*hr+3 of an A tile, at the byte positions write_digits uses.
__device__ __forceinline__ void write_fixed_digits(ATile& tile, int hr, uint32_t off,
                                                   const float (&x)[8], float S) {
  uint32_t de[kDigits], dodd[kDigits];
  fixed_digits(x[0], x[2], x[4], x[6], S, de);
  fixed_digits(x[1], x[3], x[5], x[7], S, dodd);
  uint8_t* base = &tile[4 * hr][0] + off;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes) = de[k];
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes + 8) = dodd[k];
  }
}

// Byte offset, inside row 0 of an A-operand tile, of contraction elements
// 8o..8o+7 when the B operand is fp4 in its plain order (nibble j of lane
// group g is element 32g + j): by the A byte order above, element k sits at
// byte 16(k/64) + k%16 of lane group (k%64)/16, and the octet stays whole.
__device__ __forceinline__ uint32_t a_offset_nat(int o) {
  return (uint32_t)(32 * ((o >> 1) & 3) + 16 * (o >> 3) + 8 * (o & 1));
}

// Digits of 8 values of consecutive contraction elements (bytes off..off+7
// of rows 4*hr..4*hr+3, off from a_offset_nat): the MXFP4 operands, whose B
// lane group g takes the 32 consecutive elements of block g as stored.
__device__ __forceinline__ void write_digits_nat(ATile& tile, int hr, uint32_t off,
                                                 const float (&x)[8], int eb) {
  uint32_t lo[kDigits], hi[kDigits];
  fp8_digits(x[0], x[1], x[2], x[3], eb, lo);
  fp8_digits(x[4], x[5], x[6], x[7], eb, hi);
  uint8_t* base = &tile[4 * hr][0] + off;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes) = lo[k];
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes + 4) = hi[k];
  }
}

// Fixed-point digits (fixed_digits) of 8 non-negative values of consecutive
// contraction elements, at the byte positions write_digits_nat uses.
__device__ __forceinline__ void write_fixed_digits_nat(ATile& tile, int hr, uint32_t off,
                                                       const float (&x)[8], float S) {
  uint32_t lo[kDigits], hi[kDigits];
  fixed_digits(x[0], x[1], x[2], x[3], S, lo);
  fixed_digits(x[4], x[5], x[6], x[7], S, hi);
  uint8_t* base = &tile[4 * hr][0] + off;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes) = lo[k];
    *reinterpret_cast<uint32_t*>(base + k * kRowBytes + 4) = hi[k];
  }
}

__device__ __forceinline__ v8i read_a(const ATile& tile, int m, int g) {
  const u32x4* p = reinterpret_cast<const u32x4*>(&tile[m][32 * g]);
  const u32x4 lo = p[0], hi = p[1];
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}


// ------------------------------------------------------------------ fused append
//
// With DecodeArgs::append the blocks of a head also quantize the group that
// has filled the residual window (append_common.h): its 16 items go to
// consumer waves 1..kItemWaves of the head's blocks (slot = chunk *
// kItemWaves + wave - 1), taken right after the block barrier while the
// first groups are on their way.  The step takes this path with 4 or more
// chunks per head, so a slot has at most one item.  The items run before
// the group loop, so their registers are dead by then (inside the loop they
// made the GQA-8 kernel spill).
constexpr int kItemWaves = 4;

// Channel of accumulator block blk in lane (n, r): column n of a p.V product;
// the 2-bit value words give channels 4n.. and 64 + 4n..; MXFP4 value
// columns are 16 consecutive channels.
template <bool MX>
__device__ __forceinline__ int lane_chan(int blk, int n) {
  return MX ? 16 * blk + n : 64 * (blk >> 2) + 4 * n + (blk & 3);
}

// ------------------------------------------------------------------ kernel

// MX: the cache is an MXFP4 one (kvq_mx_cache in a.c: k_codes / v_codes its
// code words, k_scale / v_scale its E8M0 bytes, no page table): keys and
// values are E2M1 codes with a power-of-two scale per block of 32 along
// each product's contraction axis, which the block-scaled matrix-core
// product takes as they are (BitDecoding page, native mxfp4 data with block
// scale factors).  The quantized part then has no per-group operand work on
// the key side (the query's digits are built once) and no min terms.
//
// PW (one chunk per consumer wave, plain 2-bit codes at GQA 4, for steps of
// many chunks): a block takes the 8 chunks c0..c0+7, the loader streams them
// interleaved (block group j is group j / 8 of chunk c0 + j % 8) and
// consumer wave w + 1 takes every group of chunk c0 + w in order, with its
// window slice.  The wave's softmax state is then its chunk's partial; the
// block merges the 8 in LDS and writes one part, so a launch of n_chunks
// chunks has n_chunks / 8 blocks and parts per head (merged in the same
// launch up to kPwFusedMergeParts of them).
template <int GQA, bool KITTY, bool MX, bool PW>
__global__ __launch_bounds__((64 * block_waves<GQA, KITTY, PW>()), 1) void decode_f8f4_kernel(DecodeArgs a) {
  static_assert(!(KITTY && MX), "the Kitty boost is a min-max cache");
  static_assert(!PW || (GQA == 4 && !KITTY && !MX), "one chunk per wave: plain 2-bit codes, GQA 4");
  constexpr int NH = GQA / 4;    // heads per lane (r and r + 4)
  constexpr int R = ring_slots<GQA, KITTY, MX, PW>();
  constexpr int DF = in_flight<GQA, KITTY, MX, PW>();
  constexpr int kWaves = block_waves<GQA, KITTY, PW>();
  // wave 0 is the loader (the first wave of a block to start), 1.. consume
  constexpr int kConsumers = kWaves - 1, kLoader = 0;
  constexpr int kThreadsF = 64 * kWaves;
  static_assert((dma_per_group<KITTY, MX>() + 1) * (DF - 1) < 64, "vmcnt range");
  static_assert(R < kSeqLen, "ready tags must not repeat within the ring");
  static_assert(sizeof(LdsF<GQA, KITTY, MX, PW>) <= 160 * 1024, "LDS per CU");
  constexpr int SB = slot_bytes<KITTY, MX>();
  constexpr int NDMA = dma_per_group<KITTY, MX>();
  __shared__ LdsF<GQA, KITTY, MX, PW> sh;

  // Every launch argument the first phase needs, fetched in one round trip
  // (the compiler would otherwise load each one just before its first use,
  // serializing several kernel-argument reads at the start of every wave).
  asm volatile("" ::"s"(a.c.k_codes), "s"(a.c.v_codes), "s"(a.c.k_scale), "s"(a.c.k_min),
               "s"(a.c.v_scale), "s"(a.c.v_min), "s"(a.c.t_cap), "s"(a.groups_per_chunk),
               "s"(a.n_groups), "s"(a.H_kv), "s"(a.H_q), "s"(a.q), "s"(a.qscale), "s"(a.n_sink), "s"(a.n_res), "s"(a.k_sink),
               "s"(a.v_sink), "s"(a.k_res), "s"(a.v_res), "s"(a.sink_cap), "s"(a.res_cap),
               "s"(a.n_chunks), "s"(a.ws), "s"(a.n_parts));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, r = lane >> 4;
  int bpart, head32;                             // head32 < 65536 (checked on the host)
  xcd_part_head(bpart, head32);
  const int64_t head = head32;
  const int b32 = head32 / a.H_kv, hk32 = head32 - b32 * a.H_kv;   // 32-bit division
  const int64_t b = b32, hk = hk32;
  const uint16_t* qrow = a.q + ((b * a.H_q) + hk * GQA) * kD;
  // the block's chunk, or (PW) its first chunk c0 and this wave's chunk
  const int c0 = PW ? bpart * kConsumers : bpart;
  const int chunk = PW ? c0 + max(wave - 1, 0) : bpart;
  const int64_t seq_g = seq_groups(a, b, kG);
  auto chunk_groups = [&](int c) -> int {   // groups of chunk c in this sequence
    const int64_t g0 = (int64_t)c * a.groups_per_chunk;
    return (int)max<int64_t>(0, min<int64_t>(seq_g, g0 + a.groups_per_chunk) - g0);
  };
  const int64_t gb = (int64_t)chunk * a.groups_per_chunk;
  const int ngc = chunk_groups(chunk);
  // this block's waves take items of the appended group (2-bit min-max cache)
  const bool app_on = !KITTY && !MX && a.append;

  // The loader wave sets up the ring's flags and meets the other waves at the
  // block barrier before its first copy; past it, the loader waits for
  // nothing but free ring slots (consumers run their fp16 window tiles after
  // the barrier, while the first groups are on their way).  Each wave passes
  // it exactly once.

  // per-wave online-softmax state (the loader's stays empty)
  float m_run[NH], l_part[NH], mterm[NH];
  float wsum[NH][8];                 // fp16-window p.V, channels of this lane
  f32x4 acc[NH][8];                  // quantized p.V: [head half][channel block], 4 digit rows
#pragma unroll
  for (int H = 0; H < NH; ++H) {
    m_run[H] = kNegInfF;
    l_part[H] = 0.f;
    mterm[H] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wsum[H][i] = 0.f;
      acc[H][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  if (wave == kLoader) {
    // ---------------------------------------------------------- loader wave
    if (tid < R) {
      sh.ready[tid] = -1;
      sh.empty[tid] = PW ? 0 : tid;   // PW: slot w's next group of chunk c0 + w
    }
    if (tid == 0) {
      sh.next_group = 0;
      sh.stalled = 0;
    }
    // the flags are written before any copy can land on them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // Copies the chunk's groups, in order, into the ring (group j -> slot
    // j % R) with DF groups in flight, and publishes each one once its data
    // is in LDS.  A slot is refilled only after a consumer copied its
    // previous group out (empty[s] == j).
    const int sub = lane & 15, part = lane >> 4;
    // Every array is a sequence of one-group blocks: the group with block
    // index blk has its key words at k_codes + 4096 blk bytes, its value words
    // at v_codes + 4096 blk, its scales and mins at + 256 blk in each of the
    // four arrays (Kitty: high-bits words + 512 blk, boosted rows + 128 blk).
    // Key words land in the slot half-token-major per 16-token tile: the 16-B
    // halves h of tokens 16t + n at 512 t + 256 h + 16 n, so a consumer's 32
    // lanes of one half read 256 contiguous bytes (token-major, their 8-B
    // reads 32 B apart hit the same banks two or four times).  Lane L of a
    // 1-KB copy takes tile L / 32, token L % 16, half (L / 16) % 2.
    const char* kp = reinterpret_cast<const char*>(a.c.k_codes) + 512 * (lane >> 5) +
                     32 * (lane & 15) + 16 * ((lane >> 4) & 1);
    const char* vp = reinterpret_cast<const char*>(a.c.v_codes) + 16 * lane;
    // metadata lanes: key scale, key min, value scale, value min (256 B each)
    const uint16_t* marr = part == 0 ? a.c.k_scale : part == 1 ? a.c.k_min
                         : part == 2 ? a.c.v_scale : a.c.v_min;
    const char* mp = reinterpret_cast<const char*>(marr) + 16 * sub;
    // Kitty lanes: 0..31 the group's 128 high-bits words, 32..39 its 128
    // boosted-row bytes (40..63 repeat them into the pad)
    const char* xp = lane < 32 ? reinterpret_cast<const char*>(a.c.k_hi) + 16 * lane
                               : reinterpret_cast<const char*>(a.c.k_bidx) + 16 * ((lane - 32) & 7);
    const int64_t xstep = lane < 32 ? kG * 4 : kD;
    // block of the head's group gi: head-major, or the page table's entry
    // (read through the constant address space: scalar loads, which the
    // vector-memory counter the copies rely on does not see)
    const int64_t pool = a.c.t_cap / kG;
    typedef __attribute__((address_space(4))) const int32_t* PagePtr;
    const PagePtr pt = a.c.pages ? (PagePtr)(uintptr_t)(a.c.pages + head * a.c.pt_stride)
                                 : (PagePtr) nullptr;
    bool bad_page = false;
    // LDS byte address of the ring (address-space cast of the generic pointer)
    const uint32_t ring0 =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)(&sh.ring[0][0]));
    // Group j goes to slot j % R with at most DF groups in flight.  Its
    // last copy is a 4-byte one from the sequence table into ready[j % R]:
    // copies land in issue order, so the slot shows j (mod kSeqLen) only
    // once the whole group is in LDS, with no publishing step in between.
    const uint32_t ready0 =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) int*)(&sh.ready[0]));
    // Blocks walk their chunks from different starting groups so that the
    // blocks streaming at the same time do not all sit at the same offsets
    // of their heads (and on the same memory channels).
    // The offsets were picked by measurement.  Plain codes: a head's chunks
    // start a quarter of a chunk apart, heads 7 groups apart (the 32K step
    // 1 us faster than with the other form, 2 us faster than with none);
    // Kitty and MXFP4 keep head * 37 + chunk * 17 (2 us faster there).
    const int rot = ngc <= 0 ? 0
                    : (KITTY || MX) ? (int)((head32 * 37 + chunk * 17) % ngc)
                                    : (int)((head32 * 7 + chunk * (ngc / 4)) % ngc);
    bool ok = true;
    // Copies group gi of the head into ring slot s, then the sequence
    // table's tag into ready[s].
    auto issue = [&](int s, int64_t gi, int tag) {
      const uint32_t sl = __builtin_amdgcn_readfirstlane(ring0 + s * SB);
      int64_t blk = head * pool + gi;
      if (pt) {
        blk = pt[gi];
        if (blk < 0 || blk >= pool) {   // a page outside the pool: copy block 0, poison
          blk = 0;
          bad_page = true;
        }
      }
      if constexpr (MX) {
        // the group's 128 tokens: key code rows (64 B each), value code rows
        // (8 tokens x 128 channels, 512 B each), key scales (4 B per token;
        // lanes 0..31) and value scales (128 B per 32 tokens; lanes 32..63)
        // (key rows land transposed: slot row 16 i + k holds token 8 k + i)
        const int64_t t0 = gi * kG;
        const char* kc = reinterpret_cast<const char*>(a.c.k_codes) + (head * a.c.t_cap + t0) * 64 +
                         512 * (lane >> 2) + 16 * (lane & 3);
        const char* vc = reinterpret_cast<const char*>(a.c.v_codes) +
                         (head * (a.c.t_cap / 8) + t0 / 8) * (kD * 4) + 16 * lane;
        const char* sc =
            lane < 32 ? reinterpret_cast<const char*>(a.c.k_scale) + (head * a.c.t_cap + t0) * 4 + 16 * lane
                      : reinterpret_cast<const char*>(a.c.v_scale) +
                            (head * (a.c.t_cap / 32) + t0 / 32) * kD + 16 * (lane - 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) dma_1k(sl + 1024 * i, kc + 64 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) dma_1k(sl + kMxV + 1024 * i, vc + 1024 * i);
        dma_1k(sl + kMxKs, sc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_1k(sl + 1024 * i, kp + blk * 4096 + 1024 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_1k(sl + kSlotV + 1024 * i, vp + blk * 4096 + 1024 * i);
        dma_1k(sl + kSlotKs, mp + blk * 256);
        if constexpr (KITTY) dma_1k(sl + kSlotHi, xp + blk * xstep);
      }
      if (lane == 0)
        dma_flag(__builtin_amdgcn_readfirstlane(ready0 + 4 * s), kSeq.v + (tag & (kSeqLen - 1)));
    };
    if constexpr (PW) {
      // One ring slot per consumer: slot w takes the groups of chunk c0 + w
      // in order, each as soon as consumer w has copied the previous one out
      // (empty[w] == its index), so a consumer that falls behind holds up
      // only its own chunk.  The loader polls the slots in turn.
      int nxt[kConsumers], ng[kConsumers];
      int left = 0;
#pragma unroll
      for (int w = 0; w < kConsumers; ++w) {
        nxt[w] = 0;
        ng[w] = chunk_groups(c0 + w);
        left += ng[w];
      }
      int issued = 0;
      uint32_t idle = 0;
      while (left > 0) {
        bool any = false;
#pragma unroll
        for (int w = 0; w < kConsumers; ++w) {
          if (nxt[w] < ng[w] && __builtin_amdgcn_readfirstlane(lds_load(&sh.empty[w])) == nxt[w]) {
            asm volatile("" ::: "memory");
            issue(w, (int64_t)(c0 + w) * a.groups_per_chunk + nxt[w], nxt[w]);
            ++nxt[w];
            --left;
            any = true;
            if (++issued >= DF) vm_wait<(NDMA + 1) * (DF - 1)>();   // at most DF - 1 in flight
          }
        }
        if (!any) {
          if (++idle >= kSpinLimit) {   // a consumer stopped taking its groups
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        } else {
          idle = 0;
        }
      }
    } else {
      for (int j = 0; j < ngc; ++j) {
        const int s = j % R;
        if (!spin_until(&sh.empty[s], j)) {
          ok = false;
          break;
        }
        asm volatile("" ::: "memory");
        issue(s, gb + (j + rot < ngc ? j + rot : j + rot - ngc), j);
        if (j >= DF - 1) vm_wait<(NDMA + 1) * (DF - 1)>();   // at most DF - 1 groups in flight
      }
    }
    vm_wait<0>();
    if ((!ok || bad_page) && lane == 0) {
      __hip_atomic_fetch_or(&sh.stalled, (ok ? 0 : 1) | (bad_page ? 2 : 0), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  } else {
    // ---------------------------------------------------------- consumer waves
    __syncthreads();   // the loader has set up the ring's flags
    // query, then this wave's first fp16 window tile (requested first, so
    // the window work waits only for them)
    u32x4 qraw[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j)
      qraw[j] = *reinterpret_cast<const u32x4*>(qrow + (r + 4 * j) * kD + 8 * n);
    // This block's slice [u0, u1) of the fp16 window (sink | residual);
    // consumer w takes 16-token tiles w, w + kConsumers, ...
    const int n_win = a.n_sink + seq_res(a, b);
    const int wpc = n_win > 0 ? (n_win + a.n_chunks - 1) / a.n_chunks : 0;
    const int u0 = min(n_win, chunk * wpc), u1 = min(n_win, u0 + wpc);
    const int kq = lane >> 4, m_row = lane & 15;
    const int cw = wave - 1;   // consumer index
    // window tiles of the wave: every kConsumers-th of the block's slice, or
    // (PW) every tile of its chunk's slice
    const int u_first = PW ? u0 : u0 + 16 * cw;
    constexpr int kWinStep = 16 * (PW ? 1 : kConsumers);
    auto win_row = [&](const uint16_t* sink, const uint16_t* res, int u) -> const uint16_t* {
      return u < a.n_sink ? sink + (head * a.sink_cap + u) * kD
                          : res + (head * a.res_cap + (u - a.n_sink)) * kD;
    };
    // one window tile: keys of token n (rows past the tile end repeat its
    // last token) and the values of token pair (lane & 7), 16-channel group
    // lane >> 3
    struct WinTile {
      u32x4 k[4];
      u32x4 v[4];
    };
    auto load_win = [&](int u, WinTile& t) {
      const int nt = min(16, u1 - u);
      const uint16_t* kr = win_row(a.k_sink, a.k_res, u + min(n, nt - 1));
#pragma unroll
      for (int c = 0; c < 4; ++c) t.k[c] = *reinterpret_cast<const u32x4*>(kr + 32 * c + 8 * kq);
      const int j = lane & 7, cg = lane >> 3;
      const uint16_t* r0 = win_row(a.v_sink, a.v_res, u + min(2 * j, nt - 1)) + 16 * cg;
      const uint16_t* r1 = win_row(a.v_sink, a.v_res, u + min(2 * j + 1, nt - 1)) + 16 * cg;
      t.v[0] = *reinterpret_cast<const u32x4*>(r0);
      t.v[1] = *reinterpret_cast<const u32x4*>(r0 + 8);
      t.v[2] = *reinterpret_cast<const u32x4*>(r1);
      t.v[3] = *reinterpret_cast<const u32x4*>(r1 + 8);
    };
    // window q.K^T A operand of this wave: rows 4h' + {hi, lo, 0, 0} of head
    // 4H + h', K-step c (channels 32c + 8kq + e), natural channel order
    u32x4 wq[NH][4];
    WinTile wt;
    if (u_first < u1) {
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          wq[H][c] = (m_row & 3) < 2 ? *reinterpret_cast<const u32x4*>(
                                           qrow + (4 * H + (m_row >> 2)) * kD + 32 * c + 8 * kq)
                                     : u32x4{0u, 0u, 0u, 0u};
      load_win(u_first, wt);
    }

    // qv[j][e] = q[r + 4j][8n + e] * sm * log2(e) * 2^(8 - e_q), |qv| < 2^8
    float qv[NH][8];
    float qmax = 0.f;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      unpack8(qraw[j], qv[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[j][e] *= a.qscale;
        qmax = fmaxf(qmax, fabsf(qv[j][e]));
      }
    }
    qmax = row_max16(qmax);
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
    const int e_q = ceil_exp(qmax);
    {
      const float qs = exp2i(8 - e_q);
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[j][e] *= qs;
    }
    const float q_unscale = exp2i(e_q - 8);
    auto chan = [&](int blk) -> int { return lane_chan<MX>(blk, n); };

    WaveLdsF<GQA, MX>& L = sh.u.w[cw];

    // ------------------------------------------------------ fp16 window
    // q.K^T on fp16 matrix cores (raw keys as B), the online softmax, p.V
    // through an LDS transpose of the fp16 values into a natural-scale
    // accumulator, reduced to the lane's channels (wsum, rescaled with the
    // softmax from here on).  The query's fp16 hi/lo rows carry the same
    // power of two as qv (largest entry below 2^8), so small entries stay
    // normal fp16 numbers with their full precision; the logits drop it again.
    if (u_first < u1) {
      const float wqs = a.qscale * exp2i(8 - e_q);
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 val = u32x4{0u, 0u, 0u, 0u};
          if ((m_row & 3) < 2) {
            float v[8];
            unpack8(wq[H][c], v);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x0 = v[2 * i] * wqs, x1 = v[2 * i + 1] * wqs;
              const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
              const auto l = __builtin_amdgcn_cvt_pkrtz(x0 - (float)h[0], x1 - (float)h[1]);
              val[i] = __builtin_bit_cast(uint32_t, (m_row & 1) ? l : h);
            }
          }
          wq[H][c] = val;
        }
      f32x4 wacc[NH][8];
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int i = 0; i < 8; ++i) wacc[H][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int u = u_first; u < u1; u += kWinStep) {
        if (u != u_first) load_win(u, wt);
        const int nt = min(16, u1 - u);
        {
          const int j = lane & 7, cg = lane >> 3;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t x = q < 4 ? wt.v[0][q] : wt.v[1][q - 4];
            const uint32_t y = q < 4 ? wt.v[2][q] : wt.v[3][q - 4];
            L.vt[16 * cg + 2 * q][j] = __builtin_amdgcn_perm(y, x, 0x05040100u);
            L.vt[16 * cg + 2 * q + 1][j] = __builtin_amdgcn_perm(y, x, 0x07060302u);
          }
        }
        const bool valid = n < nt;
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          f32x4 cw = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) cw = mfma_f16(wq[H][c], wt.k[c], cw);
          const float lg = valid ? (cw[0] + cw[1]) * q_unscale : kNegInfF;
          const float v = row_max16(lg);
          const float m_new = fmaxf(m_run[H], v);   // finite: the tile has a valid token
          const float alpha = fexp2(m_run[H] - m_new);
          m_run[H] = m_new;
          const float pw = valid ? fexp2(lg - m_new) : 0.f;
          L.p[r + 4 * H][n] = pw;
          l_part[H] = fmaf(l_part[H], alpha, pw);
#pragma unroll
          for (int i = 0; i < 8; ++i) wacc[H][i] *= alpha;
        }
        wave_sync();
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          // A = p (rows 4h' + {hi, lo, 0, 0}), tokens 8kq..8kq+7 of the tile (kq < 2)
          u32x4 apw = u32x4{0u, 0u, 0u, 0u};
          if ((m_row & 3) < 2 && kq < 2) {
            const float* pp = &L.p[4 * H + (m_row >> 2)][8 * kq];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x0 = pp[2 * i], x1 = pp[2 * i + 1];
              const auto hi = __builtin_amdgcn_cvt_pkrtz(x0, x1);
              const auto lo = __builtin_amdgcn_cvt_pkrtz(x0 - (float)hi[0], x1 - (float)hi[1]);
              apw[i] = __builtin_bit_cast(uint32_t, (m_row & 1) ? lo : hi);
            }
          }
#pragma unroll
          for (int blk = 0; blk < 8; ++blk) {
            const int d = chan(blk);
            u32x4 bv = u32x4{0u, 0u, 0u, 0u};
            if (kq < 2) {   // rows are 8-byte aligned: two 8-byte reads
              const u32x2 b0 = *reinterpret_cast<const u32x2*>(&L.vt[d][4 * kq]);
              const u32x2 b1 = *reinterpret_cast<const u32x2*>(&L.vt[d][4 * kq + 2]);
              bv = u32x4{b0[0], b0[1], b1[0], b1[1]};
            }
            wacc[H][blk] = mfma_f16(apw, bv, wacc[H][blk]);
          }
        }
        wave_sync();
      }
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int i = 0; i < 8; ++i) wsum[H][i] = wacc[H][i][0] + wacc[H][i][1];
    }

    // ------------------------------------------------------ groups
    const uint32_t a_off = a_offset(n);
    const int sa_digit = 127 - 4 * (lane & 3);   // A row m = lane & 15 holds digit m % 4
    // byte address of the lane holding the value-side exponent of this lane's
    // A-scale row (m = lane & 15) and block (g = lane >> 4)
    const int blk_src = 4 * (16 * ((lane & 15) >> 2) + 4 * (lane >> 4));
    int e_s = 0;                   // key exponent of the current group
    float bias[NH];                // its q . key-min terms
    f32x4 cq[NH][8];               // its q.K^T digit rows, per tile

    // Kitty.  The high-bits word of a token (2 bits per boosted row j,
    // rows ascending with the channel index) is the B operand of an extra
    // product; lane group g holds rows 8 (g % 2) + 2i in nibble i and rows
    // 8 (g % 2) + 2i + 1 in nibble 16 + i (i < 4), which pair with A bytes
    // 0..3 of lane groups 2 (g % 2) and 2 (g % 2) + 1 (fp4_operand, a_offset).
    // So A lane group ga, byte i must hold the q.K^T digit byte of the channel
    // of row 8 (ga / 2) + 2i + ga % 2; every other A byte is 0.  ktab (16 bytes
    // in the row padding of the first key tile) maps A byte 4 ga + i to that
    // channel's byte position in an A-tile row.
    uint8_t* const ktab = &L.op.ak[0][0][128];
    auto chan_pos = [](int c) -> uint32_t {
      return a_offset(c >> 3) + 8 * (c & 1) + ((c & 7) >> 1);
    };
    const uint32_t kpos0 = chan_pos(lane), kpos1 = chan_pos(64 + lane);
    auto ktab_slot = [](uint32_t j) -> uint32_t {
      return 8 * (j >> 3) + 4 * (j & 1) + ((j & 7) >> 1);
    };

    // copy group j's operands out of ring slot s (then the slot is free)
    auto read_slot = [&](int s, Operands& f) {
      const uint8_t* sp = &sh.ring[s][0];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x2 v =
            *reinterpret_cast<const u32x2*>(sp + 512 * t + 256 * (r >> 1) + 16 * n + 8 * (r & 1));
        f.kw[t][0] = v[0];
        f.kw[t][1] = v[1];
      }
      f.ks = *reinterpret_cast<const u32x4*>(sp + kSlotKs + 16 * n);
      f.kmin = *reinterpret_cast<const u32x4*>(sp + kSlotKm + 16 * n);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          f.vw[q][hb] = *reinterpret_cast<const u32x4*>(sp + kSlotV + (2 * r + q) * 512 +
                                                         (64 * hb + 4 * n) * 4);
      f.vs = *reinterpret_cast<const u32x4*>(sp + kSlotVs + 16 * n);
      f.vmn = *reinterpret_cast<const u32x4*>(sp + kSlotVm + 16 * n);
      if constexpr (KITTY) {
        // rows 8 (r % 2) .. 8 (r % 2) + 7 of token 16t + n
#pragma unroll
        for (int t = 0; t < 8; ++t)
          f.hw[t] = *reinterpret_cast<const uint16_t*>(sp + kSlotHi + 4 * (16 * t + n) + 2 * (r & 1));
        const uint32_t j0 = sp[kSlotBidx + lane], j1 = sp[kSlotBidx + 64 + lane];
        if (j0 < 16) ktab[ktab_slot(j0)] = (uint8_t)kpos0;
        if (j1 < 16) ktab[ktab_slot(j1)] = (uint8_t)kpos1;
      }
    };

    // key A operand of the group and its q.K^T matrix products
    auto qk_issue = [&](const Operands& pf) {
      e_s = row_exp_f16(pf.ks);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        float x[8];
        float bsum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = fmaf(qv[j][2 * i], h2f_lo(pf.ks[i]), 0.f);
          x[2 * i + 1] = fmaf(qv[j][2 * i + 1], h2f_hi(pf.ks[i]), 0.f);
          bsum = fmaf(qv[j][2 * i], h2f_lo(pf.kmin[i]), bsum);
          bsum = fmaf(qv[j][2 * i + 1], h2f_hi(pf.kmin[i]), bsum);
        }
        bias[j] = row_sum16(bsum) * q_unscale;
        write_digits(L.op.ak[j], r, a_off, x, e_s);
      }
      wave_sync();
      v8i aq[NH];
#pragma unroll
      for (int H = 0; H < NH; ++H) aq[H] = read_a(L.op.ak[H], lane & 15, lane >> 4);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v8i bk = fp4_operand(pf.kw[t][0], pf.kw[t][1]);
#pragma unroll
        for (int H = 0; H < NH; ++H)
          cq[H][t] = mfma_f8f4(aq[H], bk, f32x4{0.f, 0.f, 0.f, 0.f}, sa_digit);
      }
      if constexpr (KITTY) {
        // high bits: the codes are lo + 4 hi, so q.k gains 4 sum_j a_j hi_j
        // over the boosted rows j (block scale x4 on the digit rows)
        const uint32_t pw = *reinterpret_cast<const uint32_t*>(ktab + 4 * (lane >> 4));
        const uint32_t p0 = pw & 0xFFu, p1 = (pw >> 8) & 0xFFu, p2 = (pw >> 16) & 0xFFu,
                       p3 = pw >> 24;
        v8i ah[NH];
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          const uint8_t* row = &L.op.ak[H][lane & 15][0];
          const uint32_t dw = (uint32_t)row[p0] | ((uint32_t)row[p1] << 8) |
                              ((uint32_t)row[p2] << 16) | ((uint32_t)row[p3] << 24);
          ah[H] = v8i{(int)dw, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const v8i bh = v8i{(int)(pf.hw[t] & kNib), 0, (int)((pf.hw[t] >> 2) & kNib), 0,
                             0, 0, 0, 0};
#pragma unroll
          for (int H = 0; H < NH; ++H) cq[H][t] = mfma_f8f4(ah[H], bh, cq[H][t], sa_digit + 2);
        }
      }
    };

    // logits of the group, softmax, value A operand and p.V
    // Online softmax over a group's logits (token 16t + n of head r + 4H in
    // logit[H][t]): running max and sum, each head's rescale factor alpha,
    // and p[H][e] = the probability of token 8n + e (through an LDS transpose).
    auto softmax_group = [&](const float (&logit)[NH][8], float (&alpha)[NH], float (&p)[NH][8]) {
#pragma unroll
      for (int H = 0; H < NH; ++H) {
        float v = logit[H][0];
#pragma unroll
        for (int t = 1; t < 8; ++t) v = fmaxf(v, logit[H][t]);
        v = row_max16(v);
        // The reference moves only when the group's largest logit passes it
        // by more than kLazyMax, so most groups keep it and skip the
        // accumulators' rescale (probabilities then reach 2^kLazyMax, which
        // the fixed-point value digits and fp32 sums take as they come).
        const float m_new = v > m_run[H] + kLazyMax ? v : m_run[H];
        alpha[H] = fexp2(m_run[H] - m_new);
        m_run[H] = m_new;
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float pe = fexp2(logit[H][t] - m_new);
          if constexpr (MX) p[H][t] = pe;                  // token 8n + t
          else L.pt[r + 4 * H][16 * t + n] = pe;           // token 16t + n
          sum += pe;
        }
        l_part[H] = fmaf(l_part[H], alpha[H], sum);
      }
      // the min-max path's logits are tokens 16t + n; its p.V digits want
      // tokens 8n..8n+7 of the lane, hence a transpose through LDS (the
      // MXFP4 path loads its key rows transposed instead)
      if constexpr (!MX) {
        wave_sync();
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          const f32x4* pp = reinterpret_cast<const f32x4*>(&L.pt[r + 4 * H][8 * n]);
          const f32x4 p0 = pp[0], p1 = pp[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[H][e] = p0[e];
            p[H][4 + e] = p1[e];
          }
        }
      }
    };

    auto pv_step = [&](const Operands& pf) {
      float logit[NH][8];
      const float ek = exp2i(e_q - 8 + e_s + 1);   // fp4 codes are c/2
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          logit[H][t] =
              fmaf((cq[H][t][0] + cq[H][t][1]) + (cq[H][t][2] + cq[H][t][3]), ek, bias[H]);
      float alpha[NH];
      float p[NH][8];                // tokens 8n..8n+7 of head r + 4H
      softmax_group(logit, alpha, p);

      // value A operand: fixed-point digits of p s_t, one power of two per
      // head and 32-token block (lanes n = 4b..4b+3 of a row hold block b);
      // min term
      int sav[NH];   // the p.V product's A scale of this lane's row and block
#pragma unroll
      for (int H = 0; H < NH; ++H) {
        float x[8];
        float mt = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = fmaf(p[H][2 * i], h2f_lo(pf.vs[i]), 0.f);
          x[2 * i + 1] = fmaf(p[H][2 * i + 1], h2f_hi(pf.vs[i]), 0.f);
          mt = fmaf(p[H][2 * i], h2f_lo(pf.vmn[i]), mt);
          mt = fmaf(p[H][2 * i + 1], h2f_hi(pf.vmn[i]), mt);
        }
        mterm[H] = fmaf(mterm[H], alpha[H], mt);
        float bm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        bm = fmaxf(bm, dpp<kQuadXor1>(bm));
        bm = fmaxf(bm, dpp<kQuadXor2>(bm));
        // x < 2^eb for the whole block; blocks below 2^-100 (all but zero
        // weight) keep that exponent, so every scale stays in E8M0's range
        const int eb = max(ceil_exp(bm), -100);
        write_fixed_digits(L.op.av[H], r, a_off, x, kFixMax * exp2i(-eb));
        // row m = lane & 15 (head m / 4, digit m % 4), block g = lane >> 4:
        // the exponent of lane 16 (m / 4) + 4 g, and 2^(eb - 16) M =
        // sum_k nibble_k 2^-9 2^(eb + 5 - 4k)
        sav[H] = 132 - 4 * (lane & 3) + __builtin_amdgcn_ds_bpermute(blk_src, eb);
      }
      wave_sync();

      // rescale the accumulators by the softmax's alpha
      {
        bool same = true;
#pragma unroll
        for (int H = 0; H < NH; ++H) same = same && alpha[H] == 1.f;
        if (!__all(same)) {
#pragma unroll
          for (int H = 0; H < NH; ++H) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              acc[H][i] *= alpha[H];
              wsum[H][i] *= alpha[H];
            }
          }
        }
      }

      // p.V: one MFMA per 16-channel block and head half
#pragma unroll
      for (int H = 0; H < NH; ++H) {
        const v8i apv = read_a(L.op.av[H], lane & 15, lane >> 4);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          const int hb = blk >> 2, comp = blk & 3;
          acc[H][blk] = mfma_f8f4(apv, fp4_operand(pf.vw[0][hb][comp], pf.vw[1][hb][comp]),
                                  acc[H][blk], sav[H]);
        }
      }
    };

    // the append's items first (consumer waves 1..kItemWaves)
    if (app_on && wave - 1 < kItemWaves)
      app::run_items<2, 1>(a, head, bpart * kItemWaves + wave - 1, (int)gridDim.x * kItemWaves,
                           lane);

    // Consumers claim the chunk's groups in order from a block counter and
    // take each from the ring as soon as the loader has published it.
    // Only the claim branches on the lane; every store in the loop is made
    // by all lanes with the same value (a lane-divergent store at the end of
    // the body lets the compiler split the wave across iterations).
    if constexpr (!MX) {
      for (int it = 0;; ++it) {
        int j;
        if constexpr (PW) {   // the wave's own chunk, in order, through its own slot
          if (it >= ngc) break;
          j = it;
        } else {
          int jl = 0;
          if (lane == 0) jl = atomicAdd(&sh.next_group, 1);
          j = __builtin_amdgcn_readlane(jl, 0);
          if (j >= ngc) break;
        }
        const int s = PW ? cw : j % R;
        if (!spin_until(&sh.ready[s], j & (kSeqLen - 1))) {
          if (lane == 0) __hip_atomic_fetch_or(&sh.stalled, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          break;
        }
        asm volatile("" ::: "memory");
        Operands pf;
        read_slot(s, pf);
        asm volatile("" ::: "memory");
        // this wave's LDS reads complete in order before its next LDS write
        lds_store(&sh.empty[s], PW ? j + 1 : j + R);
        qk_issue(pf);
        pv_step(pf);
      }

      // fold the digit rows of the quantized p.V into the lane's channels
      // p.V digits carry 65535 / 65536 of p s_t, codes are c/2
      constexpr float ev = 2.f * 65536.f / 65535.f;
#pragma unroll
      for (int H = 0; H < NH; ++H) {
        const float mts = row_sum16(mterm[H]);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          const f32x4 v = acc[H][blk];
          wsum[H][blk] += fmaf((v[0] + v[1]) + (v[2] + v[3]), ev, mts);
        }
      }
    } else {
      // ---------------------------------------------------- MXFP4 groups
      // Both products on the block-scaled matrix core with the cache's codes
      // and E8M0 bytes as the B operand and its scales.  An fp4 B lane
      // (n, g) holds contraction elements 32g..32g+31 and its scale byte
      // covers them; block g of the cache (channels, resp. tokens,
      // 32g..32g+31, in order) goes to lane group g, so a lane's B operand
      // is one block as stored and its scale that block's.  The A digits
      // follow the instruction's fp8 byte order (a_offset_nat).
      //  q.K^T, tile t: column n is token 8n + t, so that a lane's eight
      //    logits (tokens 8n..8n+7) are its p.V digit bytes 8n..8n+7 in
      //    token order; lane (n, g) takes the 16 code bytes of that token,
      //    channel block g, and k_scale[8n + t][g]; A = the query's fp8
      //    digits (|qv| < 2^8), built once.
      //  p.V, channel block blk (channels 16 blk..16 blk+15): lane (n, g)
      //    takes code rows 4g..4g+3 (tokens 32g..32g+31) of channel
      //    16 blk + n and v_scale[block g][16 blk + n]; A = digits of
      //    2^8 p_t, tokens in order.
      v8i aqm[NH];
      const uint32_t a_nat = a_offset_nat(n);
#pragma unroll
      for (int H = 0; H < NH; ++H) write_digits_nat(L.op.av[H], r, a_nat, qv[H], 0);
      wave_sync();
#pragma unroll
      for (int H = 0; H < NH; ++H) aqm[H] = read_a(L.op.av[H], lane & 15, lane >> 4);
      wave_sync();   // the tile now takes the p.V digits
      for (;;) {
        int jl = 0;
        if (lane == 0) jl = atomicAdd(&sh.next_group, 1);
        const int j = __builtin_amdgcn_readlane(jl, 0);
        if (j >= ngc) break;
        const int s = j % R;
        if (!spin_until(&sh.ready[s], j & (kSeqLen - 1))) {
          if (lane == 0) __hip_atomic_fetch_or(&sh.stalled, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          break;
        }
        asm volatile("" ::: "memory");
        const uint8_t* sp = &sh.ring[s][0];
        u32x4 kc[8];
        uint32_t ksc[8], vsc[8], vc[8][4];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          kc[t] = *reinterpret_cast<const u32x4*>(sp + (16 * t + n) * 64 + 16 * r);
          ksc[t] = sp[kMxKs + (8 * n + t) * 4 + r];
        }
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vc[blk][i] = *reinterpret_cast<const uint32_t*>(sp + kMxV + (4 * r + i) * (kD * 4) +
                                                            (16 * blk + n) * 4);
          vsc[blk] = sp[kMxVs + r * kD + 16 * blk + n];
        }
        asm volatile("" ::: "memory");
        // this wave's LDS reads complete in order before its next LDS write
        lds_store(&sh.empty[s], j + R);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const v8i bk = v8i{(int)kc[t][0], (int)kc[t][1], (int)kc[t][2], (int)kc[t][3], 0, 0, 0, 0};
#pragma unroll
          for (int H = 0; H < NH; ++H)
            cq[H][t] = mfma_f8f4_mx(aqm[H], bk, f32x4{0.f, 0.f, 0.f, 0.f}, sa_digit, (int)ksc[t]);
        }
        float logit[NH][8];
#pragma unroll
        for (int H = 0; H < NH; ++H)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            logit[H][t] = ((cq[H][t][0] + cq[H][t][1]) + (cq[H][t][2] + cq[H][t][3])) * q_unscale;
        float alpha[NH];
        float p[NH][8];
        softmax_group(logit, alpha, p);
        // fixed-point digits of p, one power of two per head and 32-token
        // block (lanes n = 4b..4b+3 of a row), as on the min-max path
        int sav[NH];
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          float bm = fmaxf(fmaxf(fmaxf(p[H][0], p[H][1]), fmaxf(p[H][2], p[H][3])),
                           fmaxf(fmaxf(p[H][4], p[H][5]), fmaxf(p[H][6], p[H][7])));
          bm = fmaxf(bm, dpp<kQuadXor1>(bm));
          bm = fmaxf(bm, dpp<kQuadXor2>(bm));
          const int eb = max(ceil_exp(bm), -100);
          write_fixed_digits_nat(L.op.av[H], r, a_nat, p[H], kFixMax * exp2i(-eb));
          sav[H] = 132 - 4 * (lane & 3) + __builtin_amdgcn_ds_bpermute(blk_src, eb);
        }
        wave_sync();
        {
          bool same = true;
#pragma unroll
          for (int H = 0; H < NH; ++H) same = same && alpha[H] == 1.f;
          if (!__all(same)) {
#pragma unroll
            for (int H = 0; H < NH; ++H)
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                acc[H][i] *= alpha[H];
                wsum[H][i] *= alpha[H];
              }
          }
        }
#pragma unroll
        for (int H = 0; H < NH; ++H) {
          const v8i apv = read_a(L.op.av[H], lane & 15, lane >> 4);
#pragma unroll
          for (int blk = 0; blk < 8; ++blk)
            acc[H][blk] = mfma_f8f4_mx(apv,
                                       v8i{(int)vc[blk][0], (int)vc[blk][1], (int)vc[blk][2],
                                           (int)vc[blk][3], 0, 0, 0, 0},
                                       acc[H][blk], sav[H], (int)vsc[blk]);
        }
        wave_sync();   // the digits are read before the next group writes them
      }
      // fold the digit rows (65535 / 65536 of p) into the lane's channels
#pragma unroll
      for (int H = 0; H < NH; ++H)
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          const f32x4 v = acc[H][blk];
          wsum[H][blk] += ((v[0] + v[1]) + (v[2] + v[3])) * (65536.f / 65535.f);
        }
    }
  }

  // ---------------------------------------------------------------- block merge
  // (PW: the consumers' states are their chunks' partials; the block's part
  // is their merge, one per block of 8 chunks)
  float lsum[NH];
#pragma unroll
  for (int H = 0; H < NH; ++H) lsum[H] = row_sum16(l_part[H]);
  __syncthreads();   // the per-wave buffers are reused for the merge below
  MergeLdsF<GQA, kWaves>& M = sh.u.merge;
#pragma unroll
  for (int H = 0; H < NH; ++H) {
    const int h = r + 4 * H;
    if (n == 0) {
      M.m[wave][h] = m_run[H];
      M.l[wave][h] = lsum[H];
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      M.num[wave][h][lane_chan<MX>(blk, n)] = wsum[H][blk];
    }
  }
  __syncthreads();
  const int stall_bits = lds_load(&sh.stalled);
  const bool stalled = stall_bits != 0;
  // the reason a part is poisoned, counted in the workspace's status words
  if (tid == 0 && (stall_bits & 1)) status_add(a.status, kStatusStalled);
  if (tid == 0 && (stall_bits & 2)) status_add(a.status, kStatusBadPage);
  for (int i = tid; i < GQA * kD; i += kThreadsF) {
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
    float mm = kNegInfF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = lw[w] > 0.f ? fmaxf(mm, mw[w]) : mm;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fexp2(mw[w] - mm);
      num = lw[w] > 0.f ? fmaf(nw[w], f, num) : num;
      den = lw[w] > 0.f ? fmaf(lw[w], f, den) : den;
    }
    if (stalled) {   // a wait ran out or a page was bad: poison the part (l = 1 keeps
      num = __builtin_nanf("");   // it in the merge, acc NaN)
      den = 1.f;
      mm = 0.f;
    }
    store_record(a, (b * a.H_q) + hk * GQA + h, bpart, d, mm, den, num);
  }
  if (a.counters)
    merge_in_launch<GQA, PW ? kPwFusedMergeParts : kFusedMergeParts>(a, b, hk, head32, sh.last);

  // Kitty append (the group that has filled the residual window, Kitty page
  // 4.3 stage 3): block 0 of the head runs its 8 key items (one per wave,
  // meeting in LDS for the boosted channels' ranking), the next block (or
  // block 0 again when the head has one) its 8 value items.  At the end of
  // the blocks they delay no stream, and the head's blocks share one XCD, so
  // the items' stores into the same cache lines meet in one L2.
  if constexpr (KITTY) {
    if (a.append) {
      static_assert(block_waves<GQA, KITTY, PW>() == 8, "one Kitty item per wave");
      if (bpart == 0) {
        const int64_t gb = group_block(a.c, head, a.n_groups, kG);
        if (gb >= 0) {   // a page outside the pool: the head's group is not written
          app::KittyLds& ks = sh.u.kitty;
          const int n_hi = kG * (a.n_boost >> 4);
          app::u32x4 x[4];
          app::item_load(a, head, wave, lane, x);
          __syncthreads();   // the merge's LDS is free
          if (tid < n_hi) ks.hi[tid] = 0u;
          app::KittyKey k;
          app::kitty_stats(x, wave, lane, k, ks);
          __syncthreads();
          app::kitty_rank(wave, lane, a.n_boost, ks);
          __syncthreads();
          app::kitty_codes(a, gb, wave, lane, x, k, ks, a.n_boost);
          __syncthreads();
          if (tid < n_hi) a.c.k_hi[gb * n_hi + tid] = ks.hi[tid];
        }
      }
      if (bpart == min(1, (int)gridDim.x - 1)) {
        app::u32x4 x[4];
        app::item_load(a, head, 8 + wave, lane, x);
        app::item_store<2, true>(a, head, 8 + wave, lane, x);
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_f8f4(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.n_chunks, (unsigned)(a.B * a.H_kv));
  if (pw_decode_supported(a.n_boost, a.gqa, a.n_chunks, a.B * a.H_kv)) {
    const dim3 gpw((unsigned)(a.n_chunks / kPwChunks), (unsigned)(a.B * a.H_kv));
    decode_f8f4_kernel<4, false, false, true><<<gpw, 64 * block_waves<4, false, true>(), 0, st>>>(a);
  } else if (a.n_boost > 0) {
    if (a.gqa == 4) decode_f8f4_kernel<4, true, false, false><<<grid, 64 * block_waves<4, true>(), 0, st>>>(a);
    else decode_f8f4_kernel<8, true, false, false><<<grid, 64 * block_waves<8, true>(), 0, st>>>(a);
  } else {
    if (a.gqa == 4) decode_f8f4_kernel<4, false, false, false><<<grid, 64 * block_waves<4, false>(), 0, st>>>(a);
    else decode_f8f4_kernel<8, false, false, false><<<grid, 64 * block_waves<8, false>(), 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_mx_mfma(const kvq_mx_cache& mc, const DecodeArgs& args, hipStream_t st) {
  DecodeArgs a = args;
  a.c = CacheArgs{};
  a.c.k_codes = reinterpret_cast<uint32_t*>(mc.k_codes);
  a.c.v_codes = reinterpret_cast<uint32_t*>(mc.v_codes);
  a.c.k_scale = reinterpret_cast<uint16_t*>(mc.k_scale);   // E8M0 bytes
  a.c.v_scale = reinterpret_cast<uint16_t*>(mc.v_scale);
  a.c.t_cap = mc.t_cap;
  a.c.pages = nullptr;
  a.append = 0;
  const dim3 grid((unsigned)a.n_chunks, (unsigned)(a.B * a.H_kv));
  if (a.gqa == 4) decode_f8f4_kernel<4, false, true, false><<<grid, 64 * block_waves<4, false>(), 0, st>>>(a);
  else decode_f8f4_kernel<8, false, true, false><<<grid, 64 * block_waves<8, false>(), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
