// MXFP4 cache: quantize + pack, and dequantize (BitDecoding page, section on
// native low-precision formats: packed 4-bit data with block scale factors
// that the matrix units consume directly; the format is the OCP microscaling
// one).  A block of 32 values shares the scale 2^E, E = floor(log2 max|x|) - 2
// stored as the E8M0 byte E + 127 (-127 for a block of zeros); each value is
// the E2M1 number nearest to x / 2^E (ties to the even mantissa bit,
// magnitudes past 6 saturate), one nibble.  Blocks run along each product's
// contraction axis: 32 channels of a token for keys, 32 tokens of a channel
// for values, which is where gfx950's block-scaled matrix-core operands take
// their scales.
//
// Exactness: E comes from the fp16 bits as an integer; x / 2^E is exact in
// fp32 (fp16 inputs, |E| <= 26), and the rounding compares it with the seven
// midpoints of the E2M1 magnitudes, so no floating-point rounding is involved.

#include <hip/hip_runtime.h>

#include "kvq.h"

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E of a block from the largest magnitude's fp16 bits (sign cleared)
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  const int e = (int)(amax_bits >> 10);
  const int floor_log2 = e == 0 ? (31 - __builtin_clz(amax_bits)) - 24 : e - 15;
  return floor_log2 - 2;
}

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// E2M1 code of fp16 x in a block of exponent E.  Index i of the magnitudes
// 0, .5, 1, 1.5, 2, 3, 4, 6 counts the midpoints below |y|; at a midpoint the
// even index wins, so the comparison is > below an even index and >= below an
// odd one.
__device__ __forceinline__ uint32_t fp4_code(uint32_t x, int E) {
  const float y = fabsf(h2f(x)) * __uint_as_float((uint32_t)(127 - E) << 23);
  const uint32_t i = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) + (y > 2.5f) +
                     (y >= 3.5f) + (y > 5.0f);
  return ((x >> 12) & 8u) | i;
}

__device__ __forceinline__ float fp4_value(uint32_t code, uint32_t e8m0) {
  const float mags[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  const float m = ldexpf(mags[code & 7u], (int)e8m0 - 127);
  return (code & 8u) ? -m : m;
}

struct MxArgs {
  kvq_mx_cache c;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t src_head_stride;
  int64_t t0, n;
  int32_t n_heads;
};

// y = 0: keys, one thread per (head, token, 32-channel block);
// y = 1: values, one thread per (head, 32-token block, channel)
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(MxArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blockIdx.y == 0) {
    if (idx >= (int64_t)a.n_heads * a.n * (kD / 32)) return;
    const int c = (int)(idx % (kD / 32));
    const int64_t i = (idx / (kD / 32)) % a.n;
    const int64_t hd = idx / ((kD / 32) * a.n);
    const u32x4* src = reinterpret_cast<const u32x4*>(a.k_src + hd * a.src_head_stride +
                                                      i * kD + 32 * c);
    u32x4 x[4];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = src[j];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = max(amax, max(x[j][e] & 0x7FFFu, (x[j][e] >> 16) & 0x7FFFu));
    }
    const int E = mx_exponent(amax);
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // word j: channels 32c + 8j .. + 7
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        word |= fp4_code(x[j][e] & 0xFFFFu, E) << (8 * e);
        word |= fp4_code(x[j][e] >> 16, E) << (8 * e + 4);
      }
      w[j] = word;
    }
    const int64_t t = a.t0 + i;
    *reinterpret_cast<u32x4*>(a.c.k_codes + (hd * a.c.t_cap + t) * (kD / 8) + 4 * c) = w;
    a.c.k_scale[(hd * a.c.t_cap + t) * (kD / 32) + c] = (uint8_t)(E + 127);
  } else {
    const int64_t nb = a.n / 32;
    if (idx >= (int64_t)a.n_heads * nb * kD) return;
    const int d = (int)(idx % kD);
    const int64_t b = (idx / kD) % nb;
    const int64_t hd = idx / (kD * nb);
    const uint16_t* src = a.v_src + hd * a.src_head_stride + (32 * b) * kD + d;
    uint32_t x[32];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      x[j] = src[(int64_t)j * kD];
      amax = max(amax, x[j] & 0x7FFFu);
    }
    const int E = mx_exponent(amax);
    const int64_t w0 = a.t0 / 8 + 4 * b;   // word rows of this block's tokens
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) word |= fp4_code(x[8 * w + j], E) << (4 * j);
      a.c.v_codes[(hd * (a.c.t_cap / 8) + w0 + w) * kD + d] = (int32_t)word;
    }
    a.c.v_scale[(hd * (a.c.t_cap / 32) + a.t0 / 32 + b) * kD + d] = (uint8_t)(E + 127);
  }
}

struct MxDeqArgs {
  kvq_mx_cache c;
  int64_t t0, n;
  int32_t n_heads;
  float* k_out;
  float* v_out;
};

// one thread per (head, token, channel)
__global__ __launch_bounds__(kThreads) void mx_dequantize_kernel(MxDeqArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)a.n_heads * a.n * kD) return;
  const int d = (int)(idx % kD);
  const int64_t i = (idx / kD) % a.n;
  const int64_t hd = idx / (kD * a.n);
  const int64_t t = a.t0 + i;
  const uint32_t kw = (uint32_t)a.c.k_codes[(hd * a.c.t_cap + t) * (kD / 8) + d / 8];
  a.k_out[idx] = fp4_value((kw >> (4 * (d % 8))) & 15u,
                           a.c.k_scale[(hd * a.c.t_cap + t) * (kD / 32) + d / 32]);
  const uint32_t vw = (uint32_t)a.c.v_codes[(hd * (a.c.t_cap / 8) + t / 8) * kD + d];
  a.v_out[idx] = fp4_value((vw >> (4 * (t % 8))) & 15u,
                           a.c.v_scale[(hd * (a.c.t_cap / 32) + t / 32) * kD + d]);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvq_status check_mx_cache(const kvq_mx_cache* c) {
  if (!c || !c->k_codes || !c->k_scale || !c->v_codes || !c->v_scale) return KVQ_ERR_ARG;
  if (c->t_cap <= 0 || c->t_cap % 32) return KVQ_ERR_ARG;
  if (!aligned16(c->k_codes) || !aligned16(c->k_scale) || !aligned16(c->v_codes) ||
      !aligned16(c->v_scale))
    return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_mx_quantize_pack(const kvq_mx_cache* cache, int32_t B, int32_t H_kv,
                                           const uint16_t* k_src, const uint16_t* v_src,
                                           int64_t src_head_stride, int64_t first_token,
                                           int64_t n_tokens, void* stream) {
  kvq_status st = check_mx_cache(cache);
  if (st != KVQ_OK) return st;
  if (B <= 0 || H_kv <= 0 || first_token < 0 || n_tokens < 0) return KVQ_ERR_ARG;
  if (first_token % 32 || n_tokens % 32 || first_token + n_tokens > cache->t_cap)
    return KVQ_ERR_ARG;
  if (n_tokens == 0) return KVQ_OK;
  if (!k_src || !v_src || src_head_stride < n_tokens * kD) return KVQ_ERR_ARG;
  if (!aligned16(k_src) || !aligned16(v_src) || (src_head_stride * 2) % 16) return KVQ_ERR_ALIGN;
  const int64_t heads = (int64_t)B * H_kv;
  const int64_t work = heads * n_tokens * (kD / 32);   // the larger of the two halves
  if (heads > 0x7FFFFFFF || (work + kThreads - 1) / kThreads > 0x7FFFFFFF) return KVQ_ERR_ARG;
  MxArgs a{*cache, k_src, v_src, src_head_stride, first_token, n_tokens, (int32_t)heads};
  const dim3 grid((unsigned)((work + kThreads - 1) / kThreads), 2);
  mx_quantize_kernel<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

extern "C" kvq_status kvq_mx_dequantize(const kvq_mx_cache* cache, int32_t B, int32_t H_kv,
                                        int64_t first_token, int64_t n_tokens, float* k_out,
                                        float* v_out, void* stream) {
  kvq_status st = check_mx_cache(cache);
  if (st != KVQ_OK) return st;
  if (B <= 0 || H_kv <= 0 || first_token < 0 || n_tokens < 0 ||
      first_token + n_tokens > cache->t_cap)
    return KVQ_ERR_ARG;
  if (n_tokens == 0) return KVQ_OK;
  if (!k_out || !v_out) return KVQ_ERR_ARG;
  if (!aligned16(k_out) || !aligned16(v_out)) return KVQ_ERR_ALIGN;
  const int64_t heads = (int64_t)B * H_kv;
  const int64_t total = heads * n_tokens * kD;
  if ((total + kThreads - 1) / kThreads > 0x7FFFFFFF) return KVQ_ERR_ARG;
  MxDeqArgs a{*cache, first_token, n_tokens, (int32_t)heads, k_out, v_out};
  mx_dequantize_kernel<<<(unsigned)((total + kThreads - 1) / kThreads), kThreads, 0,
                         static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}
