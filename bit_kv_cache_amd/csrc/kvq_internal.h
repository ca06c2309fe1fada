// Internal declarations shared by the libkvq HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include "kvq.h"
#include <stdint.h>

namespace kvq {

constexpr int kD = 128;          // head dimension the kernels are built for
constexpr int kMaxGqa = 8;       // query heads per kv head
constexpr int kMaxParts = 1024;  // partials per (batch, query head) the merge accepts

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Total order key of a finite fp16 value (-0 < +0), and its inverse.
__device__ __forceinline__ uint32_t order_key(uint16_t h) {
  return (h & 0x8000u) ? (0x7FFFu - (h & 0x7FFFu)) : (0x8000u + h);
}
__device__ __forceinline__ uint16_t from_order_key(uint32_t k) {
  return (k < 0x8000u) ? (uint16_t)(0x8000u | (0x7FFFu - k)) : (uint16_t)(k - 0x8000u);
}

// ---------------------------------------------------------------- launch args

struct CacheArgs {
  uint32_t* k_codes;
  uint16_t* k_scale;
  uint16_t* k_min;
  uint32_t* k_hi;
  uint8_t* k_bidx;
  uint32_t* v_codes;
  uint16_t* v_scale;
  uint16_t* v_min;
  int64_t t_cap;
  const int32_t* pages;   // NULL: contiguous; else [heads][pt_stride] page of each group
  int64_t pt_stride;
};

// Block index of group g of head `head` in every cache array (the arrays are
// sequences of one-group blocks): head-major in a contiguous cache, the page
// table's entry in a paged one.  Returns -1 for a page outside the pool.
__device__ __forceinline__ int64_t group_block(const CacheArgs& c, int64_t head, int64_t g,
                                               int G) {
  if (!c.pages) return head * (c.t_cap / G) + g;
  const int64_t p = c.pages[head * c.pt_stride + g];
  return (p >= 0 && p < c.t_cap / G) ? p : -1;
}

struct QuantArgs {
  CacheArgs c;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t src_head_stride;
  int64_t first_group;
  int64_t n_groups;
  int32_t n_heads;
  int32_t n_boost;
  int32_t boost_score;   // Kitty channel importance: 0 range, 1 mean |x|
};

struct DequantArgs {
  CacheArgs c;
  float* k_out;
  float* v_out;
  int64_t first_group;
  int64_t n_groups;
  int32_t n_heads;
  int32_t n_boost;
};

struct DecodeArgs {
  CacheArgs c;
  const uint16_t* q;       // [B][H_q][D] fp16
  int32_t B, H_q, H_kv, gqa;
  int32_t n_boost;
  int64_t n_groups;        // quantized groups per head
  int32_t n_chunks;        // token chunks per head (parts 0..n_chunks-1)
  int32_t groups_per_chunk;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  int32_t n_sink, sink_cap;
  const uint16_t* k_res;
  const uint16_t* v_res;
  int32_t n_res, res_cap;
  float qscale;            // sm_scale * log2(e): logits kept in the log2 domain
  int32_t n_parts;         // partials per (batch, query head)
  float* ws;               // partials [B][H_q][n_parts][D+2]
  float* out;              // [B][H_q][D]
  // Arrival counters, one per (batch, kv head), zero on entry; non-null when
  // the split-K kernel merges in the same launch (the last block of a head to
  // finish merges its parts and resets the counter).
  int32_t* counters;
  // Nonzero: the split-K kernel also quantizes rows 0..G-1 of every head's
  // residual window into cache group n_groups (the streaming append).
  int32_t append;
  // Per-sequence lengths (device int32 [B], or NULL for the uniform n_groups *
  // G / n_res): quantized tokens and residual tokens of sequence b.
  const int32_t* seq_quant;
  const int32_t* seq_res;
  // Status words of the workspace (kStatusStalled, kStatusBadPage): a block
  // that poisons its part adds 1 to the word naming why.
  int32_t* status;
};

// Quantized groups and residual tokens of sequence b: the per-sequence
// lengths when given (read as scalar loads, clamped into [0, n_groups] and
// [0, n_res] so no value can move an access past the planned range), else the
// launch's uniform ones.
typedef __attribute__((address_space(4))) const int32_t* ConstI32;
__device__ __forceinline__ int64_t seq_groups(const DecodeArgs& a, int64_t b, int G) {
  if (!a.seq_quant) return a.n_groups;
  const int64_t n = ((ConstI32)(uintptr_t)a.seq_quant)[b] / G;
  return n < 0 ? 0 : (n > a.n_groups ? a.n_groups : n);
}
__device__ __forceinline__ int seq_res(const DecodeArgs& a, int64_t b) {
  if (!a.seq_res) return a.n_res;
  const int n = ((ConstI32)(uintptr_t)a.seq_res)[b];
  return n < 0 ? 0 : (n > a.n_res ? a.n_res : n);
}

// Bytes of counters at the start of a decode workspace: one arrival counter
// per (batch, kv head) for up to 65536 of them, then the status words (stalled
// blocks, parts poisoned by a bad page) and reserved space; the partials
// follow.
constexpr size_t kCounterBytes = KVQ_WS_COUNTER_BYTES;
constexpr size_t kStatusIndex = KVQ_WS_STATUS / sizeof(int32_t);
static_assert(KVQ_WS_STATUS == 65536 * sizeof(int32_t), "status words follow the counters");
constexpr int kStatusStalled = 0, kStatusBadPage = 1;

// Adds to a status word of the workspace (device-scope vector atomic, one
// lane of the calling block).
__device__ __forceinline__ void status_add(int32_t* status, int which) {
  if (status) __hip_atomic_fetch_add(status + which, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The chip hands a launch's workgroups to its 8 XCDs round-robin by linear
// id (x fastest), and each XCD has an L2 of its own.  The decode kernels
// renumber their (part, head) grid so that the parts of a head run on one
// XCD: the partial records a head's last block merges, and the cache lines
// that several parts of a head write (the appended group), then meet in one
// L2 rather than being merged in memory.  The renumbering is a bijection
// when the block count is a multiple of 8; otherwise the plain one is used.
// nblk: the blocks so numbered (the first nblk of the grid in linear order).
__device__ __forceinline__ void xcd_part_head(int& part, int& head, int nblk) {
  const int parts = (int)gridDim.x;
  if ((nblk & 7) == 0) {
    const int lin = (int)(blockIdx.x + blockIdx.y * gridDim.x);
    const int g = (lin & 7) * (nblk >> 3) + (lin >> 3);
    head = g / parts;
    part = g - head * parts;
  } else {
    part = (int)blockIdx.x;
    head = (int)blockIdx.y;
  }
}
__device__ __forceinline__ void xcd_part_head(int& part, int& head) {
  xcd_part_head(part, head, (int)(gridDim.x * gridDim.y));
}

// Parts the in-launch merge accepts (more take the merge kernel); the
// one-chunk-per-wave geometry (below), whose parts are whole blocks of 8
// chunks, accepts up to kPwFusedMergeParts.
constexpr int kFusedMergeParts = 8;
constexpr int kPwFusedMergeParts = 32;

// The matrix-core decode kernels serve GQA groups of 4 or 8 heads with
// G = 128: 2-bit codes plain or with the 16-channel Kitty boost, 4-bit codes
// plain; everything else takes the vector-ALU kernel.
inline bool mfma_decode_supported(int bits, int group, int gqa, int n_boost) {
  return group == 128 && (gqa == 4 || gqa == 8) &&
         ((bits == 2 && (n_boost == 0 || n_boost == 16)) || (bits == 4 && n_boost == 0));
}
// The 2-bit kernel's one-chunk-per-wave geometry (kPwChunks consumer waves
// per block, each with a whole chunk): plain codes at GQA 4, when the chunks
// fill every CU in one round of blocks.  It removes the per-block start and
// tail that a step of hundreds of one-chunk blocks per head pays in every
// round.  The block merges its 8 chunks' states in LDS and writes one part.
constexpr int kPwChunks = 8;
inline bool pw_decode_supported(int n_boost, int gqa, int n_chunks, int64_t heads) {
  return n_boost == 0 && gqa == 4 && n_chunks % kPwChunks == 0 &&
         n_chunks >= 4 * kPwChunks &&   // at least 4 blocks per head: the append's 16 items
         (int64_t)(n_chunks / kPwChunks) * heads >= 256;
}
inline bool pw_step(int bits, int group, int gqa, int n_boost, int n_chunks, int64_t heads) {
  return bits == 2 && mfma_decode_supported(bits, group, gqa, n_boost) &&
         pw_decode_supported(n_boost, gqa, n_chunks, heads);
}
// Parts per (batch, query head) of a decode step over n_chunks chunks: one
// per chunk, one per block of kPwChunks chunks in the one-chunk-per-wave
// geometry, one more for the fp16 window on the vector-ALU path.
inline int decode_parts(int bits, int group, int gqa, int n_boost, int n_chunks,
                        int64_t heads) {
  if (!mfma_decode_supported(bits, group, gqa, n_boost)) return n_chunks + 1;
  return pw_step(bits, group, gqa, n_boost, n_chunks, heads) ? n_chunks / kPwChunks : n_chunks;
}
// The matrix-core kernels (one part per block) merge their parts in the same
// launch when a head has at most kFusedMergeParts of them (kPwFusedMergeParts
// in the one-chunk-per-wave geometry).
inline bool fused_merge_supported(int bits, int group, int gqa, int n_boost, int n_chunks,
                                  int64_t heads) {
  if (!mfma_decode_supported(bits, group, gqa, n_boost)) return false;
  if (pw_step(bits, group, gqa, n_boost, n_chunks, heads))
    return n_chunks / kPwChunks <= kPwFusedMergeParts;
  return n_chunks <= kFusedMergeParts;
}
// The 2-bit matrix-core kernel also runs the append of a full residual group
// (plain codes, at least 4 chunks: one of the group's 16 items per consumer
// wave of the head's first four blocks, append_common.h), with the merge in
// the same launch or in a merge launch after it.  (The 4-bit kernel has no
// loader wave: items there delay every wave's first loads, and the step ran
// slower than with the append in the merge's launch.)
inline bool split_append_supported(int bits, int group, int gqa, int n_boost, int n_chunks) {
  return bits == 2 && mfma_decode_supported(bits, group, gqa, n_boost) && n_boost == 0 &&
         n_chunks >= 4;
}
// The 2-bit kernel with the 16-channel Kitty boost (boosted channels ranked
// by range) runs the append of a full residual group at the end of its
// blocks, after the in-launch merge: the 8 key items in the head's first
// block, the 8 value items in the next.
inline bool kitty_tail_append_supported(int bits, int group, int gqa, int n_boost,
                                        int boost_score, int n_chunks, int64_t heads) {
  return bits == 2 && n_boost == 16 && boost_score == 0 &&
         mfma_decode_supported(bits, group, gqa, n_boost) &&
         fused_merge_supported(bits, group, gqa, n_boost, n_chunks, heads);
}
// The 4-bit matrix-core kernel runs the append of a full residual group at
// the end of its blocks (after the in-launch merge).
inline bool tail_append_supported(int bits, int group, int gqa, int n_boost) {
  return bits == 4 && mfma_decode_supported(bits, group, gqa, n_boost);
}
// Resident blocks per CU of the matrix-core kernels: two waves per SIMD,
// as one block of 8 waves (2-bit, fp8 x fp4 kernel) or two of 4 (4-bit).
constexpr int mfma_blocks_per_cu(int bits, int) { return bits == 2 ? 1 : 2; }
constexpr int kCUs = 256;  // MI355X
inline int mfma_resident_blocks(int bits, int gqa) { return kCUs * mfma_blocks_per_cu(bits, gqa); }

// Each launcher returns the hipError_t of its launch (hipGetLastError).
// bits / v_bits: key / value code widths (equal, or the K2V4 and K4V2 pairs
// with G = 128)
hipError_t launch_quantize(int bits, int v_bits, int group, const QuantArgs& a, hipStream_t s);
hipError_t launch_dequantize(int bits, int v_bits, int group, const DequantArgs& a,
                             hipStream_t s);
hipError_t launch_decode_partials(int bits, int v_bits, int group, const DecodeArgs& a,
                                  hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);
// Split-K decode over an MXFP4 cache (vector ALU): a.n_groups counts blocks
// of 32 tokens, a.groups_per_chunk too; parts n_chunks + 1 (the last is the
// fp16 windows).
hipError_t launch_decode_mx(const kvq_mx_cache& mc, const DecodeArgs& a, hipStream_t s);
// The merge of a decode step and the quantize of an appended group (both
// small, latency-bound) as one launch; separate launches when the step has
// more than kMergeAppendParts parts.
constexpr int kMergeAppendParts = 32;
hipError_t launch_merge_append(int bits, int v_bits, int group, const DecodeArgs& d,
                               const QuantArgs& q, hipStream_t s);
hipError_t launch_decode_mfma(int bits, const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_f8f4(const DecodeArgs& a, hipStream_t s);
// Split-K decode over an MXFP4 cache on the block-scaled matrix core (GQA 4
// or 8, whole 128-token groups: a.n_groups counts them, a.groups_per_chunk
// too; parts n_chunks, the windows spread over them; merges in the same
// launch when a.counters is set).
hipError_t launch_decode_mx_mfma(const kvq_mx_cache& mc, const DecodeArgs& a, hipStream_t s);
// Whether that kernel serves an MXFP4 step.
inline bool mx_mfma_supported(int gqa, int64_t n_quant_tokens) {
  return (gqa == 4 || gqa == 8) && n_quant_tokens % 128 == 0;
}

}  // namespace kvq
