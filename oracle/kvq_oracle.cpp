// kvq oracle -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow CPU reference for the low-bit KV cache path: KIVI-style
// asymmetric min-max group quantization, bit packing, dequantization, and
// single-query decode attention in fp64 over the dequantized cache plus the
// fp16 sink/residual windows.  Only the test suite, the smoke check and the
// CPU-baseline leg of the benchmark may load this library; the product path
// never does.  It shares no code, header or table with the GPU library.
//
// Sources (the four web pages this work follows):
//  * KIVI page ("KV Cache 量化算子：KIVI"), Step 1 `quant_kcache`: per-group
//    min/max, scale = (max-min)/(2^bits-1), codes = round(clamp((x-min)/scale)).
//    Step 2 `pack_tensor`: 32/bits codes per int32, code j of a word at bit
//    bits*j (least significant first).  Step 4: unpack is (w >> bits*j) & mask,
//    dequant is code*scale + min.  Step 3: most recent tokens stay fp16.
//  * Kitty page, section 3.2/4.1/4.2 (Algorithm 1): some key channels are kept
//    at 4 bits; a key page is split into a dense 2-bit tensor with every
//    channel's low two bits, a compact 2-bit tensor with the boosted channels'
//    high two bits, and a per-channel index with a sentinel for channels that
//    are not boosted; X = lo | (hi << 2), X*scale + zero.  Section 3.1/3.3:
//    the first S tokens (sink) stay fp16.
//  * BitDecoding page, section II: attention output = softmax(Q D(K')^T) D(V').
//
// Readings where the pages are silent or inconsistent (each also listed in
// the design notes):
//  * scale denominator is 2^bits-1 (the KIVI code), not the 2^N of its prose;
//  * quantizer arithmetic: fp32 subtract, IEEE fp32 division, stored scale is
//    fp16 round-to-nearest-even, codes divide by the *stored* fp16 scale,
//    round half to even after the clamp;
//  * max == min (or a scale that underflows fp16 to zero): scale 0, codes 0,
//    dequantized value = min exactly;
//  * min/max use the total order -0 < +0 so the result never depends on the
//    reduction order;
//  * packing axis: key codes are packed along channels, value codes along
//    tokens (the contraction axis of Q.K^T and P.V respectively) with the
//    page's least-significant-first bit order;
//  * Kitty channel choice: the n_boost channels with the largest per-group
//    range (ties to the lower channel), boosted rows stored in ascending
//    channel order, sentinel = n_boost; or, by choice, the largest mean
//    magnitude over the group's tokens (section 3.2's heuristic, its T read
//    as the tokens being quantized: the page quantizes a full page at once);
//  * key and value code widths may differ (section 3.1's K2V4 and K4V2);
//  * attention covers sink + quantized + residual tokens, sm_scale defaults
//    to 1/sqrt(D), query head h reads kv head h / (H_q/H_kv).
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared (no fast-math:
// every float operation must be a single IEEE round-to-nearest-even step).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

extern "C" {

// ---------------------------------------------------------------------------
// fp16 <-> fp32.  Written from the IEEE 754 binary16 definition: 1 sign bit,
// 5 exponent bits (bias 15), 10 fraction bits; exponent field 0 encodes
// subnormals fraction * 2^-24.
// ---------------------------------------------------------------------------

double oracle_f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 31;
  const int frac = h & 1023;
  double v;
  if (expo == 0) {
    v = std::ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = std::ldexp(1.0 + frac / 1024.0, expo - 15);
  }
  return sign ? -v : v;
}

float oracle_f16_to_f32(uint16_t h) { return (float)oracle_f16_to_f64(h); }

// Round a float to the nearest binary16 value, ties to even.
uint16_t oracle_f32_to_f16(float f) {
  const uint16_t sign = std::signbit(f) ? 0x8000 : 0;
  if (std::isnan(f)) return sign | 0x7E00;
  const double a = std::fabs((double)f);
  if (std::isinf(f)) return sign | 0x7C00;
  // Binade of a, clamped to the smallest normal binade; the fp16 grid spacing
  // there is 2^(binade-10) (2^-24 for subnormals).
  int e2 = 0;
  std::frexp(a, &e2);  // a = m * 2^e2, m in [0.5, 1)
  const int binade = std::max(e2 - 1, -14);
  const double quantum = std::ldexp(1.0, binade - 10);
  // a / quantum is exact (power-of-two scaling); nearbyint rounds half to even
  // in the default rounding mode.
  const double r = std::nearbyint(a / quantum) * quantum;
  if (r >= 65536.0) return sign | 0x7C00;  // rounds past the largest finite
  uint16_t bits;
  if (r < std::ldexp(1.0, -14)) {
    bits = (uint16_t)(r / std::ldexp(1.0, -24));
  } else {
    int er = 0;
    std::frexp(r, &er);
    const int E = er - 1;
    const double frac = (r / std::ldexp(1.0, E) - 1.0) * 1024.0;
    bits = (uint16_t)(((E + 15) << 10) | (int)frac);
  }
  return sign | bits;
}

// Total order key of a finite fp16 value: -0 sorts before +0.
static uint32_t order_key(uint16_t h) {
  return (h & 0x8000) ? (uint32_t)(0x7FFF - (h & 0x7FFF)) : (uint32_t)(0x8000 + h);
}

// ---------------------------------------------------------------------------
// One quantization group (KIVI page, Step 1).
// x: n fp16 values at the given element stride.  Writes the group's fp16 min
// and fp16 scale, and (optionally) the codes.
// ---------------------------------------------------------------------------

void oracle_group_minmax(const uint16_t* x, int64_t n, int64_t stride, uint16_t* mn,
                         uint16_t* mx) {
  uint16_t lo = x[0], hi = x[0];
  for (int64_t j = 1; j < n; ++j) {
    const uint16_t v = x[j * stride];
    if (order_key(v) < order_key(lo)) lo = v;
    if (order_key(v) > order_key(hi)) hi = v;
  }
  *mn = lo;
  *mx = hi;
}

// Range of the group in fp32: f32(max) - f32(min), one rounding.
float oracle_group_range(uint16_t mn, uint16_t mx) {
  const float a = oracle_f16_to_f32(mx);
  const float b = oracle_f16_to_f32(mn);
  return a - b;
}

// scale = fp16_rne(range / maxq), the division an IEEE fp32 division.
uint16_t oracle_group_scale(uint16_t mn, uint16_t mx, int32_t maxq) {
  const float r = oracle_group_range(mn, mx);
  const float s32 = r / (float)maxq;
  return oracle_f32_to_f16(s32);
}

// code = rint(clamp((x - min) / scale, 0, maxq)); scale == 0 -> 0.
uint8_t oracle_code(uint16_t x, uint16_t mn, uint16_t s, int32_t maxq) {
  const float sf = oracle_f16_to_f32(s);
  if (sf == 0.0f) return 0;
  float y = (oracle_f16_to_f32(x) - oracle_f16_to_f32(mn)) / sf;
  if (y < 0.0f) y = 0.0f;
  if (y > (float)maxq) y = (float)maxq;
  return (uint8_t)std::nearbyint(y);
}

// Dequantized value q*scale + min in fp32.  q*scale is exact in fp32 (at most
// 8 + 11 significant bits), so this is a single rounding.
float oracle_dequant(int32_t q, uint16_t s, uint16_t mn) {
  const float prod = (float)q * oracle_f16_to_f32(s);
  return prod + oracle_f16_to_f32(mn);
}

void oracle_quantize_group(const uint16_t* x, int64_t n, int64_t stride, int32_t bits,
                           uint16_t* mn_out, uint16_t* s_out, uint8_t* codes) {
  const int32_t maxq = (1 << bits) - 1;
  uint16_t mn, mx;
  oracle_group_minmax(x, n, stride, &mn, &mx);
  const uint16_t s = oracle_group_scale(mn, mx, maxq);
  *mn_out = mn;
  *s_out = s;
  if (codes)
    for (int64_t j = 0; j < n; ++j) codes[j] = oracle_code(x[j * stride], mn, s, maxq);
}

// ---------------------------------------------------------------------------
// Bit packing (KIVI page, Step 2): word i holds codes i*fpi .. i*fpi+fpi-1,
// code j of the word at bits [bits*j, bits*j+bits).
// ---------------------------------------------------------------------------

void oracle_pack(const uint8_t* codes, int64_t n_codes, int32_t bits, uint32_t* words) {
  const int64_t fpi = 32 / bits;
  for (int64_t i = 0; i < n_codes / fpi; ++i) {
    uint32_t w = 0;
    for (int64_t j = 0; j < fpi; ++j) w |= (uint32_t)codes[i * fpi + j] << (bits * j);
    words[i] = w;
  }
}

void oracle_unpack(const uint32_t* words, int64_t n_codes, int32_t bits, uint8_t* codes) {
  const int64_t fpi = 32 / bits;
  const uint32_t mask = (bits == 32) ? 0xFFFFFFFFu : ((1u << bits) - 1u);
  for (int64_t c = 0; c < n_codes; ++c)
    codes[c] = (uint8_t)((words[c / fpi] >> (bits * (c % fpi))) & mask);
}

// ---------------------------------------------------------------------------
// The packed cache.  Per head (head = b*H_kv + h_kv), t_cap token slots; keys
// and values may use different code widths (Kitty page, section 3.1: K2V4
// and K4V2), fpi = 32/bits for keys and v_fpi = 32/v_bits for values:
//   K words  [t_cap][D/fpi]     word (t,w): channels w*fpi+j of token t
//   K scale  [t_cap/G][D] fp16  K min [t_cap/G][D] fp16
//   K hi     [t_cap][n_boost/16] word (t,w): high bits of boosted rows w*16+j
//   K bidx   [t_cap/G][D] u8    boosted row of channel d, or n_boost
//   V words  [t_cap/v_fpi][D]   word (w,d): tokens w*v_fpi+j of channel d
//   V scale  [t_cap][D/G] fp16  V min [t_cap][D/G] fp16
// ---------------------------------------------------------------------------

struct Layout {
  int32_t bits, v_bits, G, D, n_boost, score;
  int64_t t_cap, fpi, v_fpi;
  uint32_t* k_words;
  uint16_t* k_scale;
  uint16_t* k_min;
  uint32_t* k_hi;
  uint8_t* k_bidx;
  uint32_t* v_words;
  uint16_t* v_scale;
  uint16_t* v_min;

  int64_t kw(int64_t hd, int64_t t, int64_t w) const { return (hd * t_cap + t) * (D / fpi) + w; }
  int64_t km(int64_t hd, int64_t g, int64_t d) const { return (hd * (t_cap / G) + g) * D + d; }
  int64_t kh(int64_t hd, int64_t t, int64_t w) const {
    return (hd * t_cap + t) * (n_boost / 16) + w;
  }
  int64_t vw(int64_t hd, int64_t w, int64_t d) const {
    return (hd * (t_cap / v_fpi) + w) * D + d;
  }
  int64_t vm(int64_t hd, int64_t t, int64_t c) const { return (hd * t_cap + t) * (D / G) + c; }
};

// score: how the Kitty boost ranks key channels (0: range over the group,
// 1: mean magnitude over the group's tokens).
static int check_cfg(int32_t bits, int32_t v_bits, int32_t G, int32_t D, int32_t n_boost,
                     int32_t score, int64_t t_cap) {
  if (G <= 0 || D <= 0 || D % G || t_cap % G) return -1;
  for (const int32_t b : {bits, v_bits}) {
    if (b != 2 && b != 4 && b != 8) return -1;
    if (G % (32 / b) || D % (32 / b)) return -1;
  }
  if (n_boost < 0 || n_boost > D || n_boost % 16) return -1;
  if (n_boost > 0 && (bits != 2 || v_bits != 2)) return -1;   // Kitty: K2 boosted, V2
  if (score != 0 && score != 1) return -1;
  return 0;
}

#define LAYOUT(bits, v_bits, G, D, n_boost, score, t_cap)                                  \
  Layout L{bits, v_bits, G, D, n_boost, score, t_cap, 32 / (bits), 32 / (v_bits),            \
           const_cast<uint32_t*>(k_words), const_cast<uint16_t*>(k_scale),                  \
           const_cast<uint16_t*>(k_min), const_cast<uint32_t*>(k_hi),                       \
           const_cast<uint8_t*>(k_bidx), const_cast<uint32_t*>(v_words),                    \
           const_cast<uint16_t*>(v_scale), const_cast<uint16_t*>(v_min)}

// Quantize + pack one key group of one head: rows src[j*D + d], j < G.
static void quantize_key_group(const Layout& L, int64_t hd, int64_t g, const uint16_t* src) {
  const int32_t G = L.G, D = L.D;
  const int32_t maxq_lo = (1 << L.bits) - 1;
  std::vector<uint16_t> mn(D), mx(D);
  std::vector<float> range(D);
  for (int32_t d = 0; d < D; ++d) {
    oracle_group_minmax(src + d, G, D, &mn[d], &mx[d]);
    range[d] = oracle_group_range(mn[d], mx[d]);
  }
  // Kitty: the n_boost most important channels get 4-bit codes (ties to the
  // lower channel).  Importance is the channel's range over the group, or
  // (score 1) its mean magnitude over the group's tokens (Kitty page, section
  // 3.2, the magnitude heuristic s_i), ranked by the sum of |x|: the same
  // order, G being common to every channel, and exact in fp64 (each |x| is a
  // multiple of 2^-24 below 2^16, and G <= D = 128 of them need at most 47
  // significant bits).
  std::vector<double> imp(D);
  for (int32_t d = 0; d < D; ++d) {
    if (L.score == 0) {
      imp[d] = range[d];
    } else {
      double sum = 0.0;
      for (int32_t j = 0; j < G; ++j) sum += std::fabs(oracle_f16_to_f64(src[j * D + d]));
      imp[d] = sum;
    }
  }
  std::vector<int32_t> row(D, L.n_boost);
  if (L.n_boost > 0) {
    std::vector<int32_t> order(D);
    for (int32_t d = 0; d < D; ++d) order[d] = d;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return imp[a] > imp[b]; });
    std::vector<int32_t> chosen(order.begin(), order.begin() + L.n_boost);
    std::sort(chosen.begin(), chosen.end());
    for (int32_t r = 0; r < L.n_boost; ++r) row[chosen[r]] = r;
  }
  std::vector<uint8_t> codes((size_t)G * D);  // [j][d]
  for (int32_t d = 0; d < D; ++d) {
    const bool boosted = row[d] < L.n_boost;
    const int32_t maxq = boosted ? 15 : maxq_lo;
    const uint16_t s = oracle_group_scale(mn[d], mx[d], maxq);
    L.k_scale[L.km(hd, g, d)] = s;
    L.k_min[L.km(hd, g, d)] = mn[d];
    if (L.k_bidx) L.k_bidx[L.km(hd, g, d)] = (uint8_t)row[d];
    for (int32_t j = 0; j < G; ++j) codes[(size_t)j * D + d] = oracle_code(src[j * D + d], mn[d], s, maxq);
  }
  std::vector<uint8_t> lo(D);
  for (int32_t j = 0; j < G; ++j) {
    const int64_t t = g * G + j;
    for (int32_t d = 0; d < D; ++d) lo[d] = codes[(size_t)j * D + d] & maxq_lo;
    oracle_pack(lo.data(), D, L.bits, &L.k_words[L.kw(hd, t, 0)]);
    if (L.n_boost > 0) {
      std::vector<uint8_t> hi(L.n_boost);
      for (int32_t d = 0; d < D; ++d)
        if (row[d] < L.n_boost) hi[row[d]] = codes[(size_t)j * D + d] >> 2;
      oracle_pack(hi.data(), L.n_boost, 2, &L.k_hi[L.kh(hd, t, 0)]);
    }
  }
}

// Quantize + pack one value group (G tokens) of one head: per token, per
// channel group of G channels.
static void quantize_value_group(const Layout& L, int64_t hd, int64_t g, const uint16_t* src) {
  const int32_t G = L.G, D = L.D;
  std::vector<uint8_t> codes((size_t)G * D);  // [j][d]
  for (int32_t j = 0; j < G; ++j) {
    const int64_t t = g * G + j;
    for (int32_t c = 0; c < D / G; ++c) {
      uint16_t mn, s;
      oracle_quantize_group(src + (size_t)j * D + c * G, G, 1, L.v_bits, &mn, &s,
                            &codes[(size_t)j * D + c * G]);
      L.v_scale[L.vm(hd, t, c)] = s;
      L.v_min[L.vm(hd, t, c)] = mn;
    }
  }
  std::vector<uint8_t> col(L.v_fpi);
  for (int32_t d = 0; d < D; ++d)
    for (int64_t w0 = 0; w0 < G / L.v_fpi; ++w0) {
      for (int64_t j = 0; j < L.v_fpi; ++j) col[j] = codes[(size_t)(w0 * L.v_fpi + j) * D + d];
      const int64_t w = (g * G) / L.v_fpi + w0;
      oracle_pack(col.data(), L.v_fpi, L.v_bits, &L.v_words[L.vw(hd, w, d)]);
    }
}

static void run_heads(int64_t n_heads, int32_t n_threads,
                      const std::function<void(int64_t)>& fn);

// Quantize groups [first_group, first_group + n_groups) of every head from
// fp16 sources laid out [head][n_groups*G][D] with the given head stride
// (elements).  Returns 0, or -1 on a bad configuration.
int oracle_quantize_pack(int32_t bits, int32_t v_bits, int32_t G, int32_t D, int32_t n_boost,
                         int32_t score, int64_t t_cap,
                         uint32_t* k_words, uint16_t* k_scale, uint16_t* k_min, uint32_t* k_hi,
                         uint8_t* k_bidx, uint32_t* v_words, uint16_t* v_scale, uint16_t* v_min,
                         int64_t n_heads, const uint16_t* k_src, const uint16_t* v_src,
                         int64_t src_head_stride, int64_t first_group, int64_t n_groups,
                         int32_t n_threads) {
  if (check_cfg(bits, v_bits, G, D, n_boost, score, t_cap)) return -1;
  if (first_group < 0 || n_groups < 0 || (first_group + n_groups) * G > t_cap) return -1;
  LAYOUT(bits, v_bits, G, D, n_boost, score, t_cap);
  run_heads(n_heads, n_threads, [&](int64_t hd) {
    for (int64_t i = 0; i < n_groups; ++i) {
      const int64_t g = first_group + i;
      quantize_key_group(L, hd, g, k_src + hd * src_head_stride + i * G * D);
      quantize_value_group(L, hd, g, v_src + hd * src_head_stride + i * G * D);
    }
  });
  return 0;
}

// Dequantized key / value of token t, channel d (Kitty page Algorithm 1 for
// boosted key channels: X = lo | hi << 2).
static float key_at(const Layout& L, int64_t hd, int64_t t, int32_t d) {
  const int64_t g = t / L.G;
  // code d % fpi of word d / fpi (least significant first)
  const uint32_t w = L.k_words[L.kw(hd, t, d / L.fpi)];
  int32_t code = (int32_t)((w >> (L.bits * (d % L.fpi))) & ((1u << L.bits) - 1u));
  if (L.n_boost > 0) {
    const int32_t r = L.k_bidx[L.km(hd, g, d)];
    if (r < L.n_boost) {
      const uint32_t hw = L.k_hi[L.kh(hd, t, r / 16)];
      code |= (int32_t)((hw >> (2 * (r % 16))) & 3u) << 2;
    }
  }
  return oracle_dequant(code, L.k_scale[L.km(hd, g, d)], L.k_min[L.km(hd, g, d)]);
}

static float value_at(const Layout& L, int64_t hd, int64_t t, int32_t d) {
  const uint32_t w = L.v_words[L.vw(hd, t / L.v_fpi, d)];
  const int32_t q = (int32_t)((w >> (L.v_bits * (t % L.v_fpi))) & ((1u << L.v_bits) - 1u));
  const int64_t c = d / L.G;
  return oracle_dequant(q, L.v_scale[L.vm(hd, t, c)], L.v_min[L.vm(hd, t, c)]);
}

// fp32 dequantized K and V of groups [first_group, first_group+n_groups),
// written [head][n_groups*G][D].
int oracle_dequantize(int32_t bits, int32_t v_bits, int32_t G, int32_t D, int32_t n_boost,
                      int32_t score, int64_t t_cap,
                      const uint32_t* k_words, const uint16_t* k_scale, const uint16_t* k_min,
                      const uint32_t* k_hi, const uint8_t* k_bidx, const uint32_t* v_words,
                      const uint16_t* v_scale, const uint16_t* v_min, int64_t n_heads,
                      int64_t first_group, int64_t n_groups, float* k_out, float* v_out,
                      int32_t n_threads) {
  if (check_cfg(bits, v_bits, G, D, n_boost, score, t_cap)) return -1;
  if (first_group < 0 || n_groups < 0 || (first_group + n_groups) * G > t_cap) return -1;
  LAYOUT(bits, v_bits, G, D, n_boost, score, t_cap);
  const int64_t n_tok = n_groups * G;
  run_heads(n_heads, n_threads, [&](int64_t hd) {
    for (int64_t i = 0; i < n_tok; ++i) {
      const int64_t t = first_group * G + i;
      for (int32_t d = 0; d < D; ++d) {
        k_out[(hd * n_tok + i) * D + d] = key_at(L, hd, t, d);
        v_out[(hd * n_tok + i) * D + d] = value_at(L, hd, t, d);
      }
    }
  });
  return 0;
}

// ---------------------------------------------------------------------------
// Attention (BitDecoding page, section II; with the customary 1/sqrt(D)).
// One query vector against n keys/values, all fp64:
//   s_t = sm * sum_d q_d k_td,  O = sum_t e^{s_t - M} v_t / sum_t e^{s_t - M}.
// ---------------------------------------------------------------------------

void oracle_attention_fp64(const double* q, const double* K, const double* V, int64_t n,
                           int32_t D, double sm, double* out) {
  std::vector<double> s(n);
  double M = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += q[d] * K[t * D + d];
    s[t] = sm * acc;
    M = std::max(M, s[t]);
  }
  double l = 0.0;
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    const double w = std::exp(s[t] - M);
    l += w;
    for (int32_t d = 0; d < D; ++d) out[d] += w * V[t * D + d];
  }
  for (int32_t d = 0; d < D; ++d) out[d] = (n > 0) ? out[d] / l : 0.0;
}

// The same attention computed over token chunks of `chunk` tokens, each chunk
// reduced to (m, l, acc), then combined with the log-sum-exp merge.  Used only
// to check the split/merge identity.
void oracle_attention_split_merge(const double* q, const double* K, const double* V, int64_t n,
                                  int32_t D, double sm, int64_t chunk, double* out) {
  std::vector<double> ms, ls, accs;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t c1 = std::min(n, c0 + chunk);
    std::vector<double> s(c1 - c0);
    double m = -INFINITY;
    for (int64_t t = c0; t < c1; ++t) {
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d) acc += q[d] * K[t * D + d];
      s[t - c0] = sm * acc;
      m = std::max(m, s[t - c0]);
    }
    double l = 0.0;
    std::vector<double> a(D, 0.0);
    for (int64_t t = c0; t < c1; ++t) {
      const double w = std::exp(s[t - c0] - m);
      l += w;
      for (int32_t d = 0; d < D; ++d) a[d] += w * V[t * D + d];
    }
    ms.push_back(m);
    ls.push_back(l);
    accs.insert(accs.end(), a.begin(), a.end());
  }
  double M = -INFINITY;
  for (double m : ms) M = std::max(M, m);
  double L = 0.0;
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  for (size_t c = 0; c < ms.size(); ++c) {
    const double f = std::exp(ms[c] - M);
    L += ls[c] * f;
    for (int32_t d = 0; d < D; ++d) out[d] += accs[c * D + d] * f;
  }
  for (int32_t d = 0; d < D; ++d) out[d] = (n > 0) ? out[d] / L : 0.0;
}

// One decode step for every (batch, query head).  The token set of query
// head h of batch b is: n_sink fp16 sink rows, the n_quant quantized tokens
// (dequantized as above), and n_res fp16 residual rows; its kv head is
// h / (H_q / H_kv).  Windows are [head][cap][D] fp16 (either may be null
// when its count is 0).  sm <= 0 selects 1/sqrt(D).  out: [B][H_q][D] fp64.
int oracle_decode_attention(int32_t bits, int32_t v_bits, int32_t G, int32_t D, int32_t n_boost,
                            int32_t score, int64_t t_cap,
                            const uint32_t* k_words, const uint16_t* k_scale,
                            const uint16_t* k_min, const uint32_t* k_hi, const uint8_t* k_bidx,
                            const uint32_t* v_words, const uint16_t* v_scale,
                            const uint16_t* v_min, int32_t B, int32_t H_q, int32_t H_kv,
                            const uint16_t* q, int64_t n_quant, const uint16_t* k_sink,
                            const uint16_t* v_sink, int32_t n_sink, int32_t sink_cap,
                            const uint16_t* k_res, const uint16_t* v_res, int32_t n_res,
                            int32_t res_cap, double sm, double* out, int32_t n_threads) {
  if (check_cfg(bits, v_bits, G, D, n_boost, score, t_cap)) return -1;
  if (B <= 0 || H_kv <= 0 || H_q % H_kv || n_quant < 0 || n_quant % G || n_quant > t_cap)
    return -1;
  if (n_sink < 0 || n_sink > sink_cap || n_res < 0 || n_res > res_cap) return -1;
  LAYOUT(bits, v_bits, G, D, n_boost, score, t_cap);
  if (sm <= 0.0) sm = 1.0 / std::sqrt((double)D);
  const int32_t gq = H_q / H_kv;
  run_heads((int64_t)B * H_kv, n_threads, [&](int64_t hd) {
    const int64_t n = n_sink + n_quant + n_res;
    std::vector<double> K((size_t)n * D), V((size_t)n * D);
    int64_t t = 0;
    for (int32_t i = 0; i < n_sink; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = oracle_f16_to_f64(k_sink[(hd * sink_cap + i) * D + d]);
        V[t * D + d] = oracle_f16_to_f64(v_sink[(hd * sink_cap + i) * D + d]);
      }
    for (int64_t i = 0; i < n_quant; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = key_at(L, hd, i, d);
        V[t * D + d] = value_at(L, hd, i, d);
      }
    for (int32_t i = 0; i < n_res; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = oracle_f16_to_f64(k_res[(hd * res_cap + i) * D + d]);
        V[t * D + d] = oracle_f16_to_f64(v_res[(hd * res_cap + i) * D + d]);
      }
    const int64_t b = hd / H_kv, hk = hd % H_kv;
    std::vector<double> qd(D);
    for (int32_t j = 0; j < gq; ++j) {
      const int64_t h = hk * gq + j;
      for (int32_t d = 0; d < D; ++d) qd[d] = oracle_f16_to_f64(q[(b * H_q + h) * D + d]);
      oracle_attention_fp64(qd.data(), K.data(), V.data(), n, D, sm, &out[(b * H_q + h) * D]);
    }
  });
  return 0;
}

// ---------------------------------------------------------------------------
// MXFP4 cache (BitDecoding page, section on native low-precision formats: its
// Blackwell path runs the products on packed 4-bit data with block scale
// factors, mxfp4 / nvfp4; the page gives no quantizer, so the format's own
// definition is taken, the OCP microscaling one).  A block of 32 values
// shares a scale 2^E, stored as the E8M0 byte E + 127; each value is an E2M1
// number: sign, two exponent bits (bias 1, 0 = subnormal), one mantissa bit,
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  E = floor(log2(max |x|)) - 2 (2 is
// E2M1's largest exponent), so the largest magnitude lands in [4, 8) before
// rounding; every value is rounded to the nearest E2M1 magnitude, ties to
// the even mantissa bit, and magnitudes past 6 saturate to 6.  A block of
// zeros has E = -127.  Blocks run along the contraction axis of each product:
// 32 channels of one token for keys, 32 tokens of one channel for values.
//
// Layout per head, t_cap token slots (multiple of 32):
//   K codes  [t_cap][D/8] u32   nibble j of word (t,w): channel 8w + j
//   K scale  [t_cap][D/32] u8   E8M0 of channels 32c .. 32c + 31 of token t
//   V codes  [t_cap/8][D] u32   nibble j of word (w,d): token 8w + j
//   V scale  [t_cap/32][D] u8   E8M0 of tokens 32b .. 32b + 31 of channel d
// ---------------------------------------------------------------------------

static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// value of a 4-bit E2M1 code
double oracle_fp4_value(uint8_t code) {
  const double m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

// nearest E2M1 code of v (ties to the even mantissa bit, i.e. the even index;
// magnitudes past 6 saturate); the sign is v's, -0 included
uint8_t oracle_fp4_encode(double v) {
  const double a = std::fabs(v);
  int best = 0;
  for (int i = 1; i < 8; ++i) {
    const double d = std::fabs(a - kE2M1[i]), db = std::fabs(a - kE2M1[best]);
    if (d < db || (d == db && (i & 1) == 0)) best = i;
  }
  return (uint8_t)((std::signbit(v) ? 8 : 0) | best);
}

// shared exponent E of n fp16 values (stride apart)
int32_t oracle_mx_exponent(const uint16_t* x, int64_t n, int64_t stride) {
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(oracle_f16_to_f64(x[i * stride])));
  if (amax == 0.0) return -127;
  int e = 0;
  std::frexp(amax, &e);            // amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
  return std::min(127, std::max(-127, (e - 1) - 2));
}

// codes of a block with shared exponent E (x / 2^E is exact in fp64)
static void mx_block(const uint16_t* x, int64_t stride, int32_t E, uint8_t* codes) {
  for (int64_t i = 0; i < 32; ++i)
    codes[i] = oracle_fp4_encode(std::ldexp(oracle_f16_to_f64(x[i * stride]), -E));
}

// dequantized value: the E2M1 value times 2^E (exact in fp32 for fp16 inputs)
float oracle_mx_dequant(uint8_t code, uint8_t e8m0) {
  return (float)std::ldexp(oracle_fp4_value(code), (int)e8m0 - 127);
}

struct MxLayout {
  int32_t D;
  int64_t t_cap;
  uint32_t* k_words;
  uint8_t* k_scale;
  uint32_t* v_words;
  uint8_t* v_scale;
  int64_t kw(int64_t hd, int64_t t, int64_t w) const { return (hd * t_cap + t) * (D / 8) + w; }
  int64_t ks(int64_t hd, int64_t t, int64_t c) const { return (hd * t_cap + t) * (D / 32) + c; }
  int64_t vw(int64_t hd, int64_t w, int64_t d) const { return (hd * (t_cap / 8) + w) * D + d; }
  int64_t vs(int64_t hd, int64_t b, int64_t d) const { return (hd * (t_cap / 32) + b) * D + d; }
};

static float mx_key_at(const MxLayout& L, int64_t hd, int64_t t, int32_t d) {
  const uint32_t w = L.k_words[L.kw(hd, t, d / 8)];
  return oracle_mx_dequant((uint8_t)((w >> (4 * (d % 8))) & 15u), L.k_scale[L.ks(hd, t, d / 32)]);
}

static float mx_value_at(const MxLayout& L, int64_t hd, int64_t t, int32_t d) {
  const uint32_t w = L.v_words[L.vw(hd, t / 8, d)];
  return oracle_mx_dequant((uint8_t)((w >> (4 * (t % 8))) & 15u), L.v_scale[L.vs(hd, t / 32, d)]);
}

// Quantize tokens [t0, t0 + n) of every head (t0 and n multiples of 32) from
// fp16 sources [head][n][D] with the given head stride (elements).
int oracle_mx_quantize_pack(int32_t D, int64_t t_cap, uint32_t* k_words, uint8_t* k_scale,
                            uint32_t* v_words, uint8_t* v_scale, int64_t n_heads,
                            const uint16_t* k_src, const uint16_t* v_src,
                            int64_t src_head_stride, int64_t t0, int64_t n, int32_t n_threads) {
  if (D <= 0 || D % 32 || t_cap <= 0 || t_cap % 32) return -1;
  if (t0 < 0 || n < 0 || t0 % 32 || n % 32 || t0 + n > t_cap) return -1;
  MxLayout L{D, t_cap, k_words, k_scale, v_words, v_scale};
  run_heads(n_heads, n_threads, [&](int64_t hd) {
    const uint16_t* ks = k_src + hd * src_head_stride;
    const uint16_t* vs = v_src + hd * src_head_stride;
    uint8_t codes[32];
    for (int64_t i = 0; i < n; ++i)            // keys: 32 channels of a token
      for (int32_t c = 0; c < D / 32; ++c) {
        const uint16_t* x = ks + i * D + 32 * c;
        const int32_t E = oracle_mx_exponent(x, 32, 1);
        mx_block(x, 1, E, codes);
        L.k_scale[L.ks(hd, t0 + i, c)] = (uint8_t)(E + 127);
        for (int32_t w = 0; w < 4; ++w) oracle_pack(codes + 8 * w, 8, 4, &L.k_words[L.kw(hd, t0 + i, 4 * c + w)]);
      }
    for (int64_t b = 0; b < n / 32; ++b)       // values: 32 tokens of a channel
      for (int32_t d = 0; d < D; ++d) {
        const uint16_t* x = vs + (32 * b) * D + d;
        const int32_t E = oracle_mx_exponent(x, 32, D);
        mx_block(x, D, E, codes);
        L.v_scale[L.vs(hd, t0 / 32 + b, d)] = (uint8_t)(E + 127);
        for (int32_t w = 0; w < 4; ++w)
          oracle_pack(codes + 8 * w, 8, 4, &L.v_words[L.vw(hd, t0 / 8 + 4 * b + w, d)]);
      }
  });
  return 0;
}

// fp32 dequantized K and V of tokens [t0, t0 + n), written [head][n][D].
int oracle_mx_dequantize(int32_t D, int64_t t_cap, const uint32_t* k_words,
                         const uint8_t* k_scale, const uint32_t* v_words,
                         const uint8_t* v_scale, int64_t n_heads, int64_t t0, int64_t n,
                         float* k_out, float* v_out, int32_t n_threads) {
  if (D <= 0 || D % 32 || t_cap <= 0 || t_cap % 32 || t0 < 0 || n < 0 || t0 + n > t_cap)
    return -1;
  MxLayout L{D, t_cap, const_cast<uint32_t*>(k_words), const_cast<uint8_t*>(k_scale),
             const_cast<uint32_t*>(v_words), const_cast<uint8_t*>(v_scale)};
  run_heads(n_heads, n_threads, [&](int64_t hd) {
    for (int64_t i = 0; i < n; ++i)
      for (int32_t d = 0; d < D; ++d) {
        k_out[(hd * n + i) * D + d] = mx_key_at(L, hd, t0 + i, d);
        v_out[(hd * n + i) * D + d] = mx_value_at(L, hd, t0 + i, d);
      }
  });
  return 0;
}

// Decode attention over the MXFP4 cache: as oracle_decode_attention, with the
// quantized tokens [0, n_quant) dequantized as above (n_quant a multiple of 32).
int oracle_mx_decode_attention(int32_t D, int64_t t_cap, const uint32_t* k_words,
                               const uint8_t* k_scale, const uint32_t* v_words,
                               const uint8_t* v_scale, int32_t B, int32_t H_q, int32_t H_kv,
                               const uint16_t* q, int64_t n_quant, const uint16_t* k_sink,
                               const uint16_t* v_sink, int32_t n_sink, int32_t sink_cap,
                               const uint16_t* k_res, const uint16_t* v_res, int32_t n_res,
                               int32_t res_cap, double sm, double* out, int32_t n_threads) {
  if (D <= 0 || D % 32 || t_cap <= 0 || t_cap % 32) return -1;
  if (B <= 0 || H_kv <= 0 || H_q % H_kv || n_quant < 0 || n_quant % 32 || n_quant > t_cap)
    return -1;
  if (n_sink < 0 || n_sink > sink_cap || n_res < 0 || n_res > res_cap) return -1;
  MxLayout L{D, t_cap, const_cast<uint32_t*>(k_words), const_cast<uint8_t*>(k_scale),
             const_cast<uint32_t*>(v_words), const_cast<uint8_t*>(v_scale)};
  if (sm <= 0.0) sm = 1.0 / std::sqrt((double)D);
  const int32_t gq = H_q / H_kv;
  run_heads((int64_t)B * H_kv, n_threads, [&](int64_t hd) {
    const int64_t n = n_sink + n_quant + n_res;
    std::vector<double> K((size_t)n * D), V((size_t)n * D);
    int64_t t = 0;
    for (int32_t i = 0; i < n_sink; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = oracle_f16_to_f64(k_sink[(hd * sink_cap + i) * D + d]);
        V[t * D + d] = oracle_f16_to_f64(v_sink[(hd * sink_cap + i) * D + d]);
      }
    for (int64_t i = 0; i < n_quant; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = mx_key_at(L, hd, i, d);
        V[t * D + d] = mx_value_at(L, hd, i, d);
      }
    for (int32_t i = 0; i < n_res; ++i, ++t)
      for (int32_t d = 0; d < D; ++d) {
        K[t * D + d] = oracle_f16_to_f64(k_res[(hd * res_cap + i) * D + d]);
        V[t * D + d] = oracle_f16_to_f64(v_res[(hd * res_cap + i) * D + d]);
      }
    const int64_t b = hd / H_kv, hk = hd % H_kv;
    std::vector<double> qd(D);
    for (int32_t j = 0; j < gq; ++j) {
      const int64_t h = hk * gq + j;
      for (int32_t d = 0; d < D; ++d) qd[d] = oracle_f16_to_f64(q[(b * H_q + h) * D + d]);
      oracle_attention_fp64(qd.data(), K.data(), V.data(), n, D, sm, &out[(b * H_q + h) * D]);
    }
  });
  return 0;
}

}  // extern "C"

static void run_heads(int64_t n_heads, int32_t n_threads,
                      const std::function<void(int64_t)>& fn) {
  if (n_threads <= 0) n_threads = (int32_t)std::max(1u, std::thread::hardware_concurrency());
  n_threads = (int32_t)std::min<int64_t>(n_threads, std::max<int64_t>(n_heads, 1));
  if (n_threads <= 1) {
    for (int64_t hd = 0; hd < n_heads; ++hd) fn(hd);
    return;
  }
  std::vector<std::thread> pool;
  for (int32_t w = 0; w < n_threads; ++w)
    pool.emplace_back([&, w] {
      for (int64_t hd = w; hd < n_heads; hd += n_threads) fn(hd);
    });
  for (auto& th : pool) th.join();
}
