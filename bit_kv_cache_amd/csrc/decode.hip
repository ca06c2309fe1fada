// Split-K decode attention over the packed low-bit cache + fp16 windows,
// and the log-sum-exp merge of the partial results.
//
// Each block owns one (batch, kv head) and one "part": a chunk of quantized
// groups, or the fp16 sink + residual windows (workspace slot n_chunks).  It keeps, for
// every query head of the kv head's GQA group, the online-softmax state
// (running max m, running sum l, accumulator acc[D]) in the log2 domain and
// writes it to the workspace; the merge kernel combines the parts:
//   M = max_p m_p,  O = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
//
// The kernel here dequantizes in registers (code*scale + min in fp32, the
// same value the cache defines, KIVI page Step 4) and forms q.k and p.v on
// the vector ALUs.  It serves MHA and small query groups, group sizes 32/64
// and the Kitty boost; GQA groups of 4 or 8 with G = 128 go to the matrix-core
// kernel (decode_mfma.hip).  Both write the same partials.

#include "kvq_internal.h"
#include "decode_common.h"
#include "merge_common.h"

namespace kvq {
namespace {

// --------------------------------------------------------- quantized block
// Tokens [t0, t0+nt) of head `head`, nt a multiple of G, nt <= kBlockTok.
// BITS: key code width, VB: value code width.
template <int BITS, int VB, int G, int GQA>
__device__ void quant_block(const DecodeArgs& a, Lds<GQA>& s, int64_t head, int64_t t0, int nt,
                            float (&acc)[GQA]) {
  constexpr int FPI = 32 / BITS, VFPI = 32 / VB;
  constexpr uint32_t MASK = (1u << BITS) - 1u, VMASK = (1u << VB) - 1u;
  constexpr int WPT = kD / FPI;
  constexpr int NCG = kD / G;
  const int tid = threadIdx.x;
  const int64_t g0 = t0 / G;
  const int ng = nt / G;

  // the block (page) of each group, then per-group key scale/min (and Kitty
  // rows) and per-token value scale/min
  if (tid < ng) {
    const int64_t blk = group_block(a.c, head, g0 + tid, G);
    s.gblk[tid] = blk;
    if (blk < 0) s.bad = 1;
  }
  __syncthreads();
  if (s.bad) return;   // a page outside the pool: the part is poisoned
  for (int i = tid; i < ng * kD; i += kThreads) {
    const int gl = i / kD, d = i % kD;
    const int64_t off = s.gblk[gl] * kD + d;
    s.ks[gl][d] = h2f(a.c.k_scale[off]);
    s.km[gl][d] = h2f(a.c.k_min[off]);
    if (a.n_boost > 0) s.kb[gl][d] = a.c.k_bidx[off];
  }
  for (int i = tid; i < nt * NCG; i += kThreads) {
    const int t = i / NCG;
    const int64_t off = (s.gblk[t / G] * G + t % G) * NCG + i % NCG;
    s.vs[i] = h2f(a.c.v_scale[off]);
    s.vm[i] = h2f(a.c.v_min[off]);
  }
  __syncthreads();

  // q.k: thread (token t, channel half)
  {
    const int t = tid & (kBlockTok - 1), half = tid >> 7;
    if (t < nt) {
      const int gl = t / G;
      const int64_t tb = s.gblk[gl] * G + t % G;   // the token's row in the block layout
      const uint32_t* kw = a.c.k_codes + tb * WPT + half * (WPT / 2);
      uint32_t hw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (a.n_boost > 0) {
        const uint32_t* hp = a.c.k_hi + tb * (a.n_boost / 16);
        for (int w = 0; w < a.n_boost / 16; ++w) hw[w] = hp[w];
      }
      float dot[GQA];
#pragma unroll
      for (int h = 0; h < GQA; ++h) dot[h] = 0.f;
      // outer loops stay rolled: full unrolling keeps every product in
      // registers (hundreds of VGPRs, one wave per SIMD)
#pragma unroll 1
      for (int w = 0; w < WPT / 2; ++w) {
        const uint32_t word = kw[w];
#pragma unroll
        for (int j = 0; j < FPI; ++j) {
          const int c = half * (kD / 2) + w * FPI + j;
          uint32_t q = (word >> (BITS * j)) & MASK;
          if (a.n_boost > 0) {
            const int r = s.kb[gl][c];
            if (r < a.n_boost) q |= ((hw[r >> 4] >> (2 * (r & 15))) & 3u) << 2;
          }
          const float x = fmaf((float)q, s.ks[gl][c], s.km[gl][c]);
#pragma unroll
          for (int h = 0; h < GQA; ++h) dot[h] = fmaf(s.q[h][c], x, dot[h]);
        }
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

  // p.v: thread (channel d, token half)
  {
    const int d = tid & (kD - 1), half = tid >> 7;
#pragma unroll
    for (int h = 0; h < GQA; ++h) acc[h] *= s.alpha[h];
    const int tb = half * (kBlockTok / 2);
    const int te = min(nt, tb + kBlockTok / 2);
    const uint32_t* vw = a.c.v_codes + d;
    for (int tw = tb; tw < te; tw += VFPI) {
      const uint32_t word =
          __builtin_nontemporal_load(vw + ((s.gblk[tw / G] * G + tw % G) / VFPI) * kD);
#pragma unroll
      for (int j = 0; j < VFPI; ++j) {
        const int t = tw + j;
        const uint32_t q = (word >> (VB * j)) & VMASK;
        const int pi = t * NCG + d / G;
        const float x = fmaf((float)q, s.vs[pi], s.vm[pi]);
#pragma unroll
        for (int h = 0; h < GQA; ++h) acc[h] = fmaf(s.p[h][t], x, acc[h]);
      }
    }
  }
  __syncthreads();
}

// --------------------------------------------------------- MXFP4 block
typedef uint32_t mx_u32x4 __attribute__((ext_vector_type(4)));
// 2^(e8m0 - 127) for the byte range a block exponent of fp16 data can take
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return ldexpf(1.f, (int)e - 127); }

// the eight E2M1 values of a word (nibble j -> x[j], least significant
// first), each times sc, with gfx950's packed fp4 -> fp32 conversion (two
// values per instruction, the scale applied in the conversion: exact for a
// power of two)
typedef float mx_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e2m1x8(uint32_t word, float sc, float (&x)[8]) {
  const mx_f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, sc, 0);
  const mx_f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, sc, 1);
  const mx_f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, sc, 2);
  const mx_f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, sc, 3);
  x[0] = a[0], x[1] = a[1], x[2] = b[0], x[3] = b[1];
  x[4] = c[0], x[5] = c[1], x[6] = d[0], x[7] = d[1];
}

// Tokens [t0, t0+nt) of an MXFP4 cache head (t0, nt multiples of 32,
// nt <= kBlockTok): key blocks of 32 channels per token, value blocks of 32
// tokens per channel, each value E2M1 * 2^E from the hardware conversion.
template <int GQA>
__device__ void mx_block(const DecodeArgs& a, const kvq_mx_cache& mc, Lds<GQA>& s, int64_t head,
                         int64_t t0, int nt, float (&acc)[GQA]) {
  const int tid = threadIdx.x;
  // q.k: thread (token t, channel half = two key blocks)
  {
    const int t = tid & (kBlockTok - 1), half = tid >> 7;
    if (t < nt) {
      const int64_t row = head * mc.t_cap + t0 + t;
      // the token's 64 channels of this half: 8 words, two 16-byte loads
      const mx_u32x4* kw = reinterpret_cast<const mx_u32x4*>(mc.k_codes + row * (kD / 8) + 8 * half);
      float dot[GQA];
#pragma unroll
      for (int h = 0; h < GQA; ++h) dot[h] = 0.f;
#pragma unroll 1
      for (int blk = 0; blk < 2; ++blk) {
        const int c0 = 64 * half + 32 * blk;
        const float sc = e8m0_scale(mc.k_scale[row * (kD / 32) + 2 * half + blk]);
        const mx_u32x4 words = kw[blk];
#pragma unroll 1
        for (int w = 0; w < 4; ++w) {
          float x[8];
          e2m1x8(words[w], sc, x);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int h = 0; h < GQA; ++h) dot[h] = fmaf(s.q[h][c0 + 8 * w + j], x[j], dot[h]);
        }
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
  // p.v: thread (channel d, token half = two value blocks)
  {
    const int d = tid & (kD - 1), half = tid >> 7;
#pragma unroll
    for (int h = 0; h < GQA; ++h) acc[h] *= s.alpha[h];
    for (int blk = 0; blk < 2; ++blk) {
      const int tb = 64 * half + 32 * blk;   // block's first token in the tile
      if (tb >= nt) break;
      const int64_t tg = t0 + tb;
      const float sc = e8m0_scale(mc.v_scale[(head * (mc.t_cap / 32) + tg / 32) * kD + d]);
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(mc.v_codes) +
                           (head * (mc.t_cap / 8) + tg / 8) * kD + d;
#pragma unroll 1
      for (int w = 0; w < 4; ++w) {
        float x[8];
        e2m1x8(__builtin_nontemporal_load(vw + w * kD), sc, x);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int h = 0; h < GQA; ++h) acc[h] = fmaf(s.p[h][tb + 8 * w + j], x[j], acc[h]);
      }
    }
  }
  __syncthreads();
}

// grid: (n_chunks + 1, B * H_kv); part n_chunks is the fp16 windows.  A
// chunk is groups_per_chunk blocks of 32 tokens.
template <int GQA>
__global__ __launch_bounds__(kThreads) void decode_mx_kernel(DecodeArgs a, kvq_mx_cache mc) {
  __shared__ Lds<GQA> s;
  const int tid = threadIdx.x;
  int part, head32;
  xcd_part_head(part, head32);
  const int64_t head = head32;
  const int64_t b = head / a.H_kv, hk = head % a.H_kv;
  for (int i = tid; i < GQA * kD; i += kThreads) {
    const int h = i / kD, d = i % kD;
    s.q[h][d] = h2f(a.q[((b * a.H_q) + hk * GQA + h) * kD + d]) * a.qscale;
  }
  if (tid < GQA) {
    s.m[tid] = kNegInf;
    s.l[tid] = 0.f;
  }
  if (tid == 0) s.bad = 0;
  __syncthreads();
  float acc[GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) acc[h] = 0.f;
  if (part < a.n_chunks) {
    const int64_t tb = (int64_t)part * a.groups_per_chunk * 32;
    const int64_t te = min<int64_t>(a.n_groups, (int64_t)(part + 1) * a.groups_per_chunk) * 32;
    for (int64_t t = tb; t < te; t += kBlockTok)
      mx_block<GQA>(a, mc, s, head, t, (int)min<int64_t>(kBlockTok, te - t), acc);
  } else {
    const int n_win = a.n_sink + a.n_res;
    for (int u = 0; u < n_win; u += kBlockTok)
      window_block<GQA>(a, s, head, u, min(kBlockTok, n_win - u), acc);
  }
  write_partial<GQA>(a, s, b, hk, part, acc);
}

// grid: (n_chunks + 1, B * H_kv); part n_chunks is the fp16 windows
template <int BITS, int VB, int G, int GQA>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  __shared__ Lds<GQA> s;
  const int tid = threadIdx.x;
  int part, head32;
  xcd_part_head(part, head32);
  const int64_t head = head32;
  const int64_t b = head / a.H_kv, hk = head % a.H_kv;
  for (int i = tid; i < GQA * kD; i += kThreads) {
    const int h = i / kD, d = i % kD;
    s.q[h][d] = h2f(a.q[((b * a.H_q) + hk * GQA + h) * kD + d]) * a.qscale;
  }
  if (tid < GQA) {
    s.m[tid] = kNegInf;
    s.l[tid] = 0.f;
  }
  if (tid == 0) s.bad = 0;
  __syncthreads();

  float acc[GQA];
#pragma unroll
  for (int h = 0; h < GQA; ++h) acc[h] = 0.f;

  if (part < a.n_chunks) {
    const int64_t gb = (int64_t)part * a.groups_per_chunk;
    const int64_t ge = min<int64_t>(seq_groups(a, b, G), gb + a.groups_per_chunk);
    for (int64_t g = gb; g < ge && !s.bad; g += kBlockTok / G) {
      const int ng = (int)min<int64_t>(kBlockTok / G, ge - g);
      quant_block<BITS, VB, G, GQA>(a, s, head, g * G, ng * G, acc);
    }
  } else {
    const int n_win = a.n_sink + seq_res(a, b);
    for (int u = 0; u < n_win; u += kBlockTok)
      window_block<GQA>(a, s, head, u, min(kBlockTok, n_win - u), acc);
  }

  write_partial<GQA>(a, s, b, hk, part, acc);
}

// Log-sum-exp merge of up to NPM parts: one block per (batch, query head),
// one thread per channel.
template <int NPM>
__global__ __launch_bounds__(kD) void merge_small_kernel(DecodeArgs a) {
  merge_row<NPM>(a.ws, a.n_parts, a.out, blockIdx.x, threadIdx.x);
}

// Log-sum-exp merge of the parts: one block per (batch, query head).
// Parts' (m, l) are read in parallel (one per thread), the weights
// 2^(m_p - M) / L go to LDS, then thread (channel d, phase ph) sums channel d
// over the parts ph, ph + 8, ... with 16 loads in flight at a time, and the
// 8 phases' sums are added through LDS.  (The partials come from another
// launch and sit in the caches or in memory: batching the loads, rather
// than one dependent round trip per few parts, is what sets the time.)
constexpr int kMergeThreads = 1024;
constexpr int kMergePhases = kMergeThreads / kD;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a) {
  __shared__ float s_w[kMaxParts];
  __shared__ float s_red[kMergeThreads / 64];
  static_assert(kMaxParts >= kMergePhases * kD, "the phases' sums reuse s_w");
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int np = a.n_parts;
  const float* w = a.ws + bh * (int64_t)np * (kD + 2);
  // block max of the non-empty parts
  float mx = kNegInf;
  for (int p = tid; p < np; p += kMergeThreads) {
    const float l = w[p * (kD + 2) + 1];
    const float m = w[p * (kD + 2)];
    s_w[p] = l > 0.f ? m : kNegInf;
    mx = fmaxf(mx, s_w[p]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) M = fmaxf(M, s_red[i]);
  __syncthreads();
  // weights and their l-weighted sum
  float L = 0.f;
  for (int p = tid; p < np; p += kMergeThreads) {
    const float f = s_w[p] == kNegInf ? 0.f : exp2f(s_w[p] - M);
    s_w[p] = f;
    L = fmaf(w[p * (kD + 2) + 1], f, L);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  if (lane == 0) s_red[wave] = L;
  __syncthreads();
  float Ls = 0.f;
#pragma unroll
  for (int i = 0; i < kMergeThreads / 64; ++i) Ls += s_red[i];
  // numerators: thread (channel d, phase ph), 16 independent loads at a time
  const int d = tid & (kD - 1), ph = tid / kD;
  float o = 0.f;
  int p = ph;
  for (; p + kMergePhases * 15 < np; p += kMergePhases * 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = w[(p + kMergePhases * j) * (kD + 2) + 2 + d];
#pragma unroll
    for (int j = 0; j < 16; ++j) o = fmaf(v[j], s_w[p + kMergePhases * j], o);
  }
  for (; p < np; p += kMergePhases) o = fmaf(w[p * (kD + 2) + 2 + d], s_w[p], o);
  __syncthreads();
  s_w[ph * kD + d] = o;   // s_w is free again: the phases' sums
  __syncthreads();
  if (ph == 0) {
    float t = s_w[d];
#pragma unroll
    for (int q = 1; q < kMergePhases; ++q) t += s_w[q * kD + d];
    a.out[bh * kD + d] = Ls > 0.f ? t / Ls : 0.f;
  }
}

template <int BITS, int VB, int G>
hipError_t decode_bg(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_chunks + 1), (unsigned)(a.B * a.H_kv));
  switch (a.gqa) {
    case 1: decode_valu_kernel<BITS, VB, G, 1><<<grid, kThreads, 0, st>>>(a); break;
    case 2: decode_valu_kernel<BITS, VB, G, 2><<<grid, kThreads, 0, st>>>(a); break;
    case 4: decode_valu_kernel<BITS, VB, G, 4><<<grid, kThreads, 0, st>>>(a); break;
    case 8: decode_valu_kernel<BITS, VB, G, 8><<<grid, kThreads, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// equal widths for every group size, the mixed pairs for G = 128 only
template <int BITS, int VB>
hipError_t decode_bits(int group, const DecodeArgs& a, hipStream_t st) {
  if constexpr (VB != BITS) {
    return group == 128 ? decode_bg<BITS, VB, 128>(a, st) : hipErrorInvalidValue;
  } else {
    switch (group) {
      case 32: return decode_bg<BITS, VB, 32>(a, st);
      case 64: return decode_bg<BITS, VB, 64>(a, st);
      case 128: return decode_bg<BITS, VB, 128>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
}

}  // namespace

hipError_t launch_decode_partials(int bits, int v_bits, int group, const DecodeArgs& a,
                                  hipStream_t st) {
  if (bits != v_bits) {
    if (bits == 2 && v_bits == 4) return decode_bits<2, 4>(group, a, st);
    if (bits == 4 && v_bits == 2) return decode_bits<4, 2>(group, a, st);
    return hipErrorInvalidValue;
  }
  return mfma_decode_supported(bits, group, a.gqa, a.n_boost)
             ? launch_decode_mfma(bits, a, st)
             : (bits == 2   ? decode_bits<2, 2>(group, a, st)
                : bits == 4 ? decode_bits<4, 4>(group, a, st)
                            : decode_bits<8, 8>(group, a, st));
}

hipError_t launch_decode_mx(const kvq_mx_cache& mc, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_chunks + 1), (unsigned)(a.B * a.H_kv));
  switch (a.gqa) {
    case 1: decode_mx_kernel<1><<<grid, kThreads, 0, st>>>(a, mc); break;
    case 2: decode_mx_kernel<2><<<grid, kThreads, 0, st>>>(a, mc); break;
    case 4: decode_mx_kernel<4><<<grid, kThreads, 0, st>>>(a, mc); break;
    case 8: decode_mx_kernel<8><<<grid, kThreads, 0, st>>>(a, mc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.B * a.H_q);
  if (a.n_parts <= 8) merge_small_kernel<8><<<blocks, kD, 0, st>>>(a);
  else if (a.n_parts <= 16) merge_small_kernel<16><<<blocks, kD, 0, st>>>(a);
  else if (a.n_parts <= 32) merge_small_kernel<32><<<blocks, kD, 0, st>>>(a);
  else merge_kernel<<<blocks, kMergeThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
