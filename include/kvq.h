/*
 * kvq.h -- C ABI of libkvq, a low-bit KV cache for single-query decode
 * attention on AMD Instinct MI355X (gfx950).
 *
 * What it computes
 *  - KIVI-style asymmetric min-max group quantization (KIVI page, Step 1):
 *    for a group x of G values, mn = min x, scale = fp16((max x - mn)/(2^bits-1)),
 *    code = round(clamp((x - mn)/scale, 0, 2^bits-1)).  Keys are grouped per
 *    channel over G consecutive tokens, values per token over G consecutive
 *    channels (KIVI page, Step 1: K per-channel, V per-token).
 *  - Packing 32/bits codes per 32-bit word, code j at bits [bits*j, bits*j+bits)
 *    (KIVI page, Step 2 `pack_tensor`; unpack in Step 4).
 *  - Optional Kitty channel-wise precision boost (Kitty page, sections 3.2,
 *    4.1, 4.2): per key group the n_boost channels with the largest range use
 *    4-bit codes, stored as a dense tensor of every channel's low two bits, a
 *    compact tensor of the boosted channels' high two bits and a per-channel
 *    index (sentinel = n_boost); dequantization is (lo | hi << 2)*scale + min.
 *  - Single-query decode attention softmax(q K^T * sm) V (BitDecoding page,
 *    section II) over: an fp16 sink window (Kitty page, section 3.1), the
 *    quantized tokens (dequantized on chip), and an fp16 residual window of
 *    the most recent tokens (KIVI page, Step 3), split over token chunks with
 *    an fp32 log-sum-exp merge.
 *
 * Arithmetic contract (identical on every path, checked against a CPU oracle)
 *  - quantizer: fp32 range max-min, IEEE fp32 division by 2^bits-1, scale
 *    rounded to fp16 (nearest even); codes divide by the stored fp16 scale in
 *    IEEE fp32, clamp, then round half to even; max == min (or a scale that
 *    underflows fp16) stores scale 0 and codes 0.  min/max use the order
 *    -0 < +0.  Packed words, scales, mins, high words and indices are
 *    bit-exact.
 *  - dequantized value: fp32 code*scale + min (one rounding).
 *  - attention: fp32, output fp32; max-abs error vs an fp64 reference over
 *    the same dequantized cache within 2e-3 for the documented inputs.
 *
 * Cache layout (device memory owned by the caller).  head = b*H_kv + h,
 * fpi = 32/bits (keys), v_fpi = 32/v_bits (values), D = head_dim, G = group,
 * t_cap = token capacity per head:
 *    k_codes  [head][t_cap][D/fpi]       key codes packed along channels:
 *                                        word (t,w) holds channels w*fpi+j
 *    k_scale, k_min [head][t_cap/G][D]   fp16 bits per (group, channel)
 *    k_hi     [head][t_cap][n_boost/16]  Kitty: word (t,w) holds the high two
 *                                        bits of boosted rows w*16+j
 *    k_bidx   [head][t_cap/G][D] uint8   Kitty: boosted row of channel d
 *                                        (ascending channel order) or n_boost
 *    v_codes  [head][t_cap/v_fpi][D]     value codes packed along tokens:
 *                                        word (w,d) holds tokens w*v_fpi+j
 *    v_scale, v_min [head][t_cap][D/G]   fp16 bits per (token, channel group)
 *  Keys are packed along the channel axis and values along the token axis:
 *  the contraction axis of q.K^T and p.V, so one word feeds one lane's
 *  matrix-core operand directly.
 *  Every array above is a sequence of per-group blocks: group g of head h is
 *  block h*(t_cap/G) + g.
 *
 * Paged layout (Kitty page, section 4.1: a page holds one group of tokens;
 * PagedAttention-style serving).  With cache.page_table != NULL the arrays
 * are a pool of t_cap/G one-group pages laid out as the blocks above, and
 * group g of head h lives in page page_table[h*pt_stride + g].  Every call
 * reads (and the quantize calls write) only the table entries of the groups
 * it touches; an entry outside [0, t_cap/G) is never dereferenced: the
 * quantize calls skip that group and the decode calls return NaN for that
 * head's query rows.
 *
 * Conventions
 *  - fp16 data is passed as raw uint16_t bit patterns.
 *  - All pointers except `cfg`/`cache`/window structs themselves are device
 *    pointers, 16-byte aligned (else KVQ_ERR_ALIGN).
 *  - `stream` is a hipStream_t (NULL = default stream).  Calls are
 *    asynchronous; nothing synchronizes the host.
 *  - The library allocates no memory and keeps no state between calls.
 *  - Every argument is validated before anything is launched; on error
 *    nothing is launched or written.  A failed launch returns KVQ_ERR_HIP.
 *  - Non-finite inputs give undefined results.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,         /* bad size, null pointer, out-of-range index */
  KVQ_ERR_ALIGN = -2,       /* a device pointer is not 16-byte aligned */
  KVQ_ERR_UNSUPPORTED = -3, /* legal for the method, not built (D != 128, G not 32/64/128, ...) */
  KVQ_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  KVQ_ERR_HIP = -5          /* a kernel launch failed */
} kvq_status;

/* Quantization configuration.
 *  bits: 2, 4 or 8 (the KIVI page's packing widths).  8-bit codes take the
 *        vector-ALU decode kernel.
 *  group: G, one of 32, 64, 128; must divide head_dim.
 *  head_dim: D, 128.
 *  n_boost: 0 (plain KIVI) or, with bits == 2, a multiple of 16 up to D
 *        (Kitty boost; 16 of 128 channels is the 12.5% "Kitty" setting).
 *  v_bits: width of the value codes, 0 for the key width `bits`.  Mixed
 *        widths are the Kitty page's K2V4 and K4V2 variants (section 3.1):
 *        bits 2 with v_bits 4 or bits 4 with v_bits 2, G = 128 only (other
 *        mixes: KVQ_ERR_UNSUPPORTED); they take the vector-ALU decode kernel.
 *        With n_boost > 0, v_bits must be 0 or 2.
 *  boost_score: how the Kitty boost ranks a group's key channels: 0 by range
 *        (max - min over the group), 1 by mean magnitude over the group's
 *        tokens (Kitty page, section 3.2's heuristic); ties go to the lower
 *        channel.  Ignored when n_boost == 0. */
typedef struct kvq_qcfg {
  int32_t bits;
  int32_t group;
  int32_t head_dim;
  int32_t n_boost;
  int32_t v_bits;
  int32_t boost_score;
} kvq_qcfg;

/* Packed cache, layout above.  k_hi / k_bidx may be NULL when n_boost == 0.
 * t_cap must be a positive multiple of G.
 *  page_table: NULL (contiguous: t_cap tokens per head) or device int32
 *      [heads][pt_stride] (paged: t_cap/G pages in the pool); pt_stride must
 *      cover every group a call touches. */
typedef struct kvq_cache {
  int32_t* k_codes;
  uint16_t* k_scale;
  uint16_t* k_min;
  int32_t* k_hi;
  uint8_t* k_bidx;
  int32_t* v_codes;
  uint16_t* v_scale;
  uint16_t* v_min;
  int64_t t_cap;
  const int32_t* page_table;
  int64_t pt_stride;
} kvq_cache;

/* An fp16 window of full-precision tokens (sink or residual): k and v are
 * [head][cap][D] fp16, the first n rows of each head are valid.  k/v may be
 * NULL when n == 0. */
typedef struct kvq_window {
  const uint16_t* k;
  const uint16_t* v;
  int32_t n;
  int32_t cap;
} kvq_window;

/* Human-readable name of a status code (static storage). */
const char* kvq_status_string(kvq_status s);

/* Quantize and pack groups [first_group, first_group + n_groups) of every
 * head (KIVI page Steps 1-2; Kitty page section 4.1 when n_boost > 0).
 *  k_src, v_src: fp16 [B*H_kv][>= n_groups*G][D]; head i starts at element
 *      i*src_head_stride.  Typically the residual window (append one full
 *      group after a decode step, Kitty page section 4.3 stage 3) or a
 *      prefill slab (n_groups > 1).
 *  Writes codes, scales, mins (and Kitty high words / indices) of those
 *  groups only.  Requires (first_group + n_groups)*G <= t_cap and
 *  src_head_stride >= n_groups*G*D.  n_groups == 0 is a no-op. */
kvq_status kvq_quantize_pack(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                             int32_t H_kv, const uint16_t* k_src, const uint16_t* v_src,
                             int64_t src_head_stride, int64_t first_group, int64_t n_groups,
                             void* stream);

/* Split plan of a decode step: the number of token chunks per head
 * (n_chunks_req > 0 is honoured up to one chunk per group and at most 1023;
 * 0 picks a count that fills the GPU) and the workspace size in bytes it needs. */
kvq_status kvq_decode_plan(const kvq_qcfg* cfg, int32_t B, int32_t H_q, int32_t H_kv,
                           int64_t n_quant_tokens, int32_t n_chunks_req, int32_t* n_chunks,
                           size_t* ws_bytes);

/* Decode workspace layout: KVQ_WS_COUNTER_BYTES of int32 counters, then the
 * fp32 partial records.  The counter bytes are
 *   [0, 262144)       arrival counters, one per (batch, kv head);
 *   KVQ_WS_STATUS     int32 status[2]:
 *     status[0]  blocks of a decode launch whose bounded wait for another
 *                wave of the block ran out (the block then stops waiting and
 *                poisons its part: NaN output for that head's query rows);
 *                never expected, a symptom of a scheduling fault;
 *     status[1]  parts poisoned because a page-table entry lay outside the
 *                pool (an input error; NaN output for that head);
 *   the rest up to KVQ_WS_COUNTER_BYTES is reserved (zero).
 * The counter bytes must be zero when a workspace is first used (allocate it
 * zeroed).  Every call leaves the arrival counters zero, so a workspace stays
 * valid across calls and configurations; the status words only grow (device-
 * scope atomic adds), so the caller reads them after a call and clears them
 * when it wants a fresh count.  The records need no initialization.  Calls
 * that share a workspace must not overlap in time. */
#define KVQ_WS_COUNTER_BYTES 262400
#define KVQ_WS_STATUS 262144

/* Workspace bytes of kvq_decode_attention for the same arguments (0 on a bad
 * argument): the counter bytes plus fp32 partials (m, l, acc[D]) per (batch,
 * query head, part). */
size_t kvq_decode_workspace_bytes(const kvq_qcfg* cfg, int32_t B, int32_t H_q, int32_t H_kv,
                                  int64_t n_quant_tokens, int32_t n_chunks_req);

/* One decode step (BitDecoding page, section II: single-query attention over
 * a low-bit cache; KIVI page, Step 4: the quantized keys and values read as
 * code*scale + min; Kitty page, section 4.2, Algorithm 1 for boosted key
 * channels; KIVI page, Step 3 and Kitty page, section 3.1 for the fp16
 * windows): for batch b and query head h (kv head h / (H_q/H_kv)),
 *   out[b][h] = softmax(sm * q[b][h] . K^T) V
 * over the sink window, the first n_quant_tokens cached tokens and the
 * residual window (which holds the current token).  Split-K over token
 * chunks, the chunks combined by the log-sum-exp identity (the merge of
 * kvq_decode_merge).
 *  q: fp16 [B][H_q][D].  out: fp32 [B][H_q][D].
 *  n_quant_tokens: multiple of G, 0 <= n_quant_tokens <= t_cap.
 *  sink, res: may be NULL (no tokens).
 *  sm_scale <= 0 selects 1/sqrt(D).
 *  n_chunks: token chunks per head for split-K (0 = automatic); see
 *      kvq_decode_plan.  workspace: device memory of at least
 *      kvq_decode_workspace_bytes(...) bytes, 16-byte aligned, counter bytes
 *      zero (layout above).
 *  H_q / H_kv must be 1..8.
 *  The matrix-core kernels (2-bit codes plain or with 16 boosted channels,
 *  4-bit codes; G = 128, GQA 4 or 8) with at most 8 parts per head, and the
 *  one-chunk-per-wave geometry (below) with at most 32, run as one launch:
 *  the last block of each head to finish merges the head's partial records
 *  (device-scope stores and loads, one arrival counter per head); other
 *  configurations launch the merge separately. */
kvq_status kvq_decode_attention(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                int32_t H_q, int32_t H_kv, const uint16_t* q,
                                int64_t n_quant_tokens, const kvq_window* sink,
                                const kvq_window* res, float sm_scale, int32_t n_chunks,
                                void* workspace, size_t ws_bytes, float* out, void* stream);

/* One decode step with the streaming append: the attention of
 * kvq_decode_attention (same arguments and result) and, when append != 0, the
 * quantize + pack of the first G rows of the residual window of every head
 * into cache group n_quant_tokens / G -- the residual group that has filled
 * up (KIVI page, Step 3; Kitty page, section 4.3, stage 3), whose tokens this
 * step still attends to in fp16.  The cache contents equal those of
 * kvq_quantize_pack(cfg, cache, B, H_kv, res->k, res->v, res->cap * D,
 * n_quant_tokens / G, 1), bit for bit.  With G = 128 and GQA 4 or 8, plain
 * 2-bit codes with at least 4 chunks and 4-bit codes quantize the group in
 * the split-K launch (16 items per head, taken by the head's blocks: 2-bit
 * before their group loops, 4-bit after their merge): when the merge runs in
 * place (as for kvq_decode_attention) the whole step is that one launch,
 * otherwise a merge launch follows.  2-bit codes with 16 boosted channels
 * ranked by range do the same when the merge runs in place (the head's first
 * block runs the 8 key items after the merge, the next block the 8 value
 * items).  Otherwise the quantization shares the merge's launch (separate
 * launches past 32 parts).
 *  append != 0 requires res->n >= G and n_quant_tokens + G <= t_cap
 *  (else KVQ_ERR_ARG, nothing launched). */
kvq_status kvq_decode_step(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_q,
                           int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                           const kvq_window* sink, const kvq_window* res, float sm_scale,
                           int32_t n_chunks, void* workspace, size_t ws_bytes, float* out,
                           int32_t append, void* stream);

/* kvq_decode_step for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, result and kernels, without the workspace.  The workspace
 * is an array of KVQ_NOALLOC_SCRATCH_BYTES in the library's code object, one
 * per GPU, held until the process ends; the call uses the array of the
 * current device (the stream must belong to it) and allocates nothing.
 * Each call first zeroes its heads' arrival counters and the status words
 * (two small kernels on `stream`), then runs the step.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialized by the caller.
 * Errors: as kvq_decode_step; KVQ_ERR_WORKSPACE when the step needs more
 * than KVQ_NOALLOC_SCRATCH_BYTES of workspace (KVQ_WS_COUNTER_BYTES plus
 * B*H_q*parts*(D+2)*4: up to 15,627 (batch, query head, part) records), with
 * nothing launched. */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
kvq_status kvq_decode_step_noalloc(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                   int32_t H_q, int32_t H_kv, const uint16_t* q,
                                   int64_t n_quant_tokens, const kvq_window* sink,
                                   const kvq_window* res, float sm_scale, int32_t n_chunks,
                                   float* out, int32_t append, void* stream);

/* The two phases of kvq_decode_attention, for callers that combine partial
 * results of several calls (for example a sequence split across devices, each
 * holding a token range of the same heads) or time the phases apart.
 *
 * kvq_decode_partials: the split-K phase (same arguments as
 * kvq_decode_attention, no output).  Writes, for every batch b, query head h
 * and part p < *n_parts, the fp32 record (rec = workspace + counter bytes)
 *     rec[((b*H_q + h)*n_parts + p)*(D+2) + {0, 1, 2..D+1}]
 *         = m, l, acc[0..D-1]
 * of one token range (BitDecoding page, section II; the combination rule is
 * the log-sum-exp merge): with x_t = sm*log2(e)*(q . k_t) over the range's
 * tokens, m = max x_t, l = sum 2^(x_t - m), acc = sum 2^(x_t - m) v_t.  An
 * empty range has l = 0 (m is then meaningless).  *n_parts receives the
 * number of parts per (b, h): the chunk count of kvq_decode_plan; an eighth
 * of it in the one-chunk-per-wave geometry (plain 2-bit codes, G = 128,
 * GQA 4, a chunk count that is a multiple of 8, at least 32, with at least
 * 256 blocks of 8 chunks over all heads), whose parts are the merged states
 * of 8 consecutive chunks; one more (the fp16 windows) on the vector-ALU path
 * (GQA 1 or 2, G != 128, 8-bit codes, n_boost other than 0 or 16, or keys
 * and values at different widths).
 *
 * kvq_decode_merge: out[b][h] = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
 * over the parts with l_p > 0 (M the largest such m_p); 0 when every part is
 * empty.  This is the log-sum-exp identity: the softmax over the union of the
 * parts' tokens (BitDecoding page, section II, normalizes over the whole
 * sequence) rebuilt from each part's max, sum and weighted value sum.  Reads workspace laid out as above with 1 <= n_parts <= 1024 and
 * ws_bytes >= KVQ_WS_COUNTER_BYTES + B*H_q*n_parts*(D+2)*4.  Neither call
 * touches the counter bytes. */
kvq_status kvq_decode_partials(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                               int32_t H_q, int32_t H_kv, const uint16_t* q,
                               int64_t n_quant_tokens, const kvq_window* sink,
                               const kvq_window* res, float sm_scale, int32_t n_chunks,
                               void* workspace, size_t ws_bytes, int32_t* n_parts,
                               void* stream);

kvq_status kvq_decode_merge(int32_t B, int32_t H_q, int32_t n_parts, const float* workspace,
                            size_t ws_bytes, float* out, void* stream);

/* Ragged batches: kvq_decode_attention and kvq_decode_partials where sequence
 * b attends to its own number of cached and residual tokens (serving with
 * sequences of different lengths, typically with a paged cache).
 *  seq_quant_tokens: device int32 [B] or NULL: quantized tokens of sequence b
 *      (rounded down to a multiple of G, clamped into [0, n_quant_tokens]);
 *      n_quant_tokens is the batch's maximum and sizes the split-K plan.
 *  seq_res_tokens: device int32 [B] or NULL: residual tokens of sequence b
 *      (clamped into [0, res->n]).
 * Everything else as in the uniform calls; the clamps keep every access
 * inside the uniform call's range whatever the arrays hold. */
kvq_status kvq_decode_attention_ragged(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                       int32_t H_q, int32_t H_kv, const uint16_t* q,
                                       int64_t n_quant_tokens, const kvq_window* sink,
                                       const kvq_window* res, const int32_t* seq_quant_tokens,
                                       const int32_t* seq_res_tokens, float sm_scale,
                                       int32_t n_chunks, void* workspace, size_t ws_bytes,
                                       float* out, void* stream);

kvq_status kvq_decode_partials_ragged(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                      int32_t H_q, int32_t H_kv, const uint16_t* q,
                                      int64_t n_quant_tokens, const kvq_window* sink,
                                      const kvq_window* res, const int32_t* seq_quant_tokens,
                                      const int32_t* seq_res_tokens, float sm_scale,
                                      int32_t n_chunks, void* workspace, size_t ws_bytes,
                                      int32_t* n_parts, void* stream);

/* Dequantize groups [first_group, first_group + n_groups) of every head to
 * fp32 [B*H_kv][n_groups*G][D] (value = code*scale + min; Kitty page
 * Algorithm 1 for boosted key channels).  For checking the packed cache. */
kvq_status kvq_dequantize(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_kv,
                          int64_t first_group, int64_t n_groups, float* k_out, float* v_out,
                          void* stream);

/* MXFP4 cache (BitDecoding page, section on native low-precision formats:
 * mxfp4 / nvfp4 data with block scale factors in the layout the matrix units
 * take; the format is the OCP microscaling one).  D = 128.  A block of 32
 * values shares the scale 2^E, E = floor(log2 max|x|) - 2, stored as the E8M0
 * byte E + 127 (a block of zeros: E = -127); each value is the nearest E2M1
 * number to x / 2^E (0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign; ties to the even
 * mantissa bit; magnitudes past 6 saturate), one nibble, least significant
 * first.  Blocks run along each product's contraction axis.  Per head
 * (b*H_kv + h), t_cap token slots (a multiple of 32):
 *    k_codes  [head][t_cap][D/8]    nibble j of word (t,w): channel 8w+j
 *    k_scale  [head][t_cap][D/32]   E8M0 of channels 32c..32c+31 of token t
 *    v_codes  [head][t_cap/8][D]    nibble j of word (w,d): token 8w+j
 *    v_scale  [head][t_cap/32][D]   E8M0 of tokens 32b..32b+31 of channel d
 * Caller-owned device memory, 16-byte aligned. */
typedef struct kvq_mx_cache {
  int32_t* k_codes;
  uint8_t* k_scale;
  int32_t* v_codes;
  uint8_t* v_scale;
  int64_t t_cap;
} kvq_mx_cache;

/* Quantize tokens [first_token, first_token + n_tokens) of every head
 * (both multiples of 32) from fp16 [head][n_tokens][D] with the given head
 * stride (elements, a multiple of 8).  Writes those tokens' codes and
 * scales only.  Errors: KVQ_ERR_ARG (bad sizes or range), KVQ_ERR_ALIGN. */
kvq_status kvq_mx_quantize_pack(const kvq_mx_cache* cache, int32_t B, int32_t H_kv,
                                const uint16_t* k_src, const uint16_t* v_src,
                                int64_t src_head_stride, int64_t first_token, int64_t n_tokens,
                                void* stream);

/* Dequantize tokens [first_token, first_token + n_tokens) of every head to
 * fp32 [head][n_tokens][D] (value = E2M1 value * 2^E, exact).  For checking
 * the packed cache. */
kvq_status kvq_mx_dequantize(const kvq_mx_cache* cache, int32_t B, int32_t H_kv,
                             int64_t first_token, int64_t n_tokens, float* k_out, float* v_out,
                             void* stream);

/* Decode attention over an MXFP4 cache: the same result as
 * kvq_decode_attention (sink | tokens [0, n_quant_tokens) | residual, fp32
 * output), the quantized keys and values read as E2M1 value * 2^E.
 * n_quant_tokens a multiple of 32 (0 allowed).  With GQA 4 or 8 and
 * n_quant_tokens a multiple of 128 the split-K kernel runs both products on
 * the block-scaled matrix cores (the E2M1 codes as the B operand and the E8M0
 * bytes as its block scales, the query and probabilities as fp8 digit rows),
 * one part per chunk, the fp16 windows shared among the chunks, merged in the
 * same launch when there are at most 8 chunks (as kvq_decode_attention);
 * otherwise the vector-ALU kernel runs over chunks of 32-token blocks plus a
 * window part, followed by the merge launch.  kvq_mx_decode_plan gives the
 * chunk count (n_chunks_req = 0: automatic; n_chunks_req > 0 is honoured up
 * to one chunk per 128-token group on the matrix-core path, at most 1023,
 * and one per 32-token block on the vector-ALU path) and the workspace size
 * (the counter bytes, then B*H_q*parts*(D+2) fp32 partials, parts = chunks
 * on the matrix-core path and chunks + 1 otherwise); errors as
 * kvq_decode_attention. */
kvq_status kvq_mx_decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int64_t n_quant_tokens,
                              int32_t n_chunks_req, int32_t* n_chunks, size_t* ws_bytes);
kvq_status kvq_mx_decode_attention(const kvq_mx_cache* cache, int32_t B, int32_t H_q,
                                   int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                                   const kvq_window* sink, const kvq_window* res, float sm_scale,
                                   int32_t n_chunks, void* workspace, size_t ws_bytes, float* out,
                                   void* stream);

/* Measurement aid, not part of the method: read `bytes` bytes at `src` once
 * (16-byte loads, `blocks` workgroups of `threads` lanes, each workgroup a
 * contiguous slice) and write nothing but a word that depends on every byte
 * into `sink` when it equals an improbable value.  Timing it over the same
 * bytes as a decode step gives the bandwidth that a plain read reaches on the
 * chip, the practical ceiling of the decode kernels, which stream every byte
 * of the cache once.  mode 0: ordinary loads; mode 1: non-temporal loads.
 * src 16-byte aligned and bytes a multiple of 16 (else KVQ_ERR_ALIGN);
 * threads a multiple of 64 in [64, 1024], blocks in [1, 2^20], sink holding
 * blocks*threads words (else KVQ_ERR_ARG). */
kvq_status kvq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                           int32_t threads, int32_t mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
