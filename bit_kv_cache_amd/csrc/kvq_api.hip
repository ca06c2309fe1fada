// Host side of the libkvq C ABI: argument validation (pure host code, run
// before anything touches the GPU), split planning and kernel launch.

#include <math.h>

#include <algorithm>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

using kvq::kD;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Value code width (0 in the configuration: the key width).
int vbits(const kvq_qcfg* cfg) { return cfg->v_bits ? cfg->v_bits : cfg->bits; }
// The code width the matrix-core and fused kernels are chosen by: the key
// width when keys and values share it, else 0 (no such kernel).
int same_bits(const kvq_qcfg* cfg) { return vbits(cfg) == cfg->bits ? cfg->bits : 0; }

// Checks shared by every entry point.
kvq_status check_cfg(const kvq_qcfg* cfg) {
  if (!cfg) return KVQ_ERR_ARG;
  if (cfg->head_dim > 0 && cfg->head_dim != kD) return KVQ_ERR_UNSUPPORTED;
  if (cfg->bits != 2 && cfg->bits != 4 && cfg->bits != 8) return KVQ_ERR_ARG;
  if (cfg->head_dim != kD) return KVQ_ERR_ARG;
  const int fpi = 32 / cfg->bits;
  if (cfg->group <= 0 || cfg->group % fpi || kD % cfg->group) return KVQ_ERR_ARG;
  if (cfg->group != 32 && cfg->group != 64 && cfg->group != 128) return KVQ_ERR_UNSUPPORTED;
  if (cfg->n_boost < 0 || cfg->n_boost > kD || cfg->n_boost % 16) return KVQ_ERR_ARG;
  if (cfg->n_boost > 0 && cfg->bits != 2) return KVQ_ERR_ARG;
  const int vb = vbits(cfg);
  if (vb != 2 && vb != 4 && vb != 8) return KVQ_ERR_ARG;
  if (cfg->group % (32 / vb)) return KVQ_ERR_ARG;
  if (cfg->n_boost > 0 && vb != 2) return KVQ_ERR_ARG;   // Kitty values are 2-bit
  if (cfg->boost_score != 0 && cfg->boost_score != 1) return KVQ_ERR_ARG;
  if (vb != cfg->bits) {   // the mixed widths built: K2V4 and K4V2 with G = 128
    if (!((cfg->bits == 2 && vb == 4) || (cfg->bits == 4 && vb == 2))) return KVQ_ERR_UNSUPPORTED;
    if (cfg->group != 128) return KVQ_ERR_UNSUPPORTED;
  }
  return KVQ_OK;
}

kvq_status check_cache(const kvq_qcfg* cfg, const kvq_cache* c) {
  if (!c) return KVQ_ERR_ARG;
  if (c->t_cap <= 0 || c->t_cap % cfg->group) return KVQ_ERR_ARG;
  if (!c->k_codes || !c->k_scale || !c->k_min || !c->v_codes || !c->v_scale || !c->v_min)
    return KVQ_ERR_ARG;
  if (cfg->n_boost > 0 && (!c->k_hi || !c->k_bidx)) return KVQ_ERR_ARG;
  if (!aligned16(c->k_codes) || !aligned16(c->k_scale) || !aligned16(c->k_min) ||
      !aligned16(c->v_codes) || !aligned16(c->v_scale) || !aligned16(c->v_min))
    return KVQ_ERR_ALIGN;
  if (cfg->n_boost > 0 && (!aligned16(c->k_hi) || !aligned16(c->k_bidx))) return KVQ_ERR_ALIGN;
  if (c->page_table && (c->pt_stride <= 0 || (reinterpret_cast<uintptr_t>(c->page_table) & 3u)))
    return c->pt_stride <= 0 ? KVQ_ERR_ARG : KVQ_ERR_ALIGN;
  return KVQ_OK;
}

kvq::CacheArgs cache_args(const kvq_cache* c) {
  return {reinterpret_cast<uint32_t*>(c->k_codes), c->k_scale, c->k_min,
          reinterpret_cast<uint32_t*>(c->k_hi), c->k_bidx,
          reinterpret_cast<uint32_t*>(c->v_codes), c->v_scale, c->v_min, c->t_cap,
          c->page_table, c->page_table ? c->pt_stride : 0};
}

// The groups [0, end_group) of every head must be addressable: in a
// contiguous cache within t_cap, in a paged one within the table's rows.
bool groups_fit(const kvq_cache* c, int64_t G, int64_t end_group) {
  return c->page_table ? end_group <= c->pt_stride : end_group * G <= c->t_cap;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// Chunks per head.  Vector-ALU kernel: enough blocks to give every compute
// unit several (the fp16 windows are one more block per head).  Matrix-core
// kernel: the resident block slots divided over the heads, so the grid runs
// in a single round (windows are spread over the chunks; at least one chunk).
// An explicit request is honoured up to one chunk per group (and 1023).
constexpr int64_t kMaxChunks = kvq::kMaxParts - 1;  // plus the window part

int32_t plan_chunks(bool mfma, int bits, int gqa, int64_t heads, int64_t n_groups, int32_t req) {
  int64_t n;
  if (req > 0) {
    n = req;
  } else if (mfma) {
    n = kvq::mfma_resident_blocks(bits, gqa) / heads;
  } else {
    const int64_t target_blocks = 1024;  // 256 CUs x 4
    n = (target_blocks + heads - 1) / heads;
  }
  if (n > n_groups) n = n_groups;
  if (n > kMaxChunks) n = kMaxChunks;
  if (n < 1) n = mfma ? 1 : (n_groups > 0 ? 1 : 0);
  return (int32_t)n;
}

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Workspace: fp32 partials [B][H_q][parts][D+2].  Parts are the chunks, plus
// the fp16-window part on the vector-ALU kernel (the matrix-core kernel
// spreads the windows over its chunks).
size_t partial_bytes(int64_t B, int64_t H_q, int64_t parts) {
  return align16((size_t)B * H_q * parts * (kD + 2) * sizeof(float));
}

// Workspace: arrival counters (zero between calls), then the partials.
size_t workspace_bytes(int64_t B, int64_t H_q, int64_t parts) {
  return kvq::kCounterBytes + partial_bytes(B, H_q, parts);
}

kvq_status check_window(const kvq_window* w) {
  if (!w) return KVQ_OK;
  if (w->n < 0 || w->cap < 0 || w->n > w->cap) return KVQ_ERR_ARG;
  if (w->n > 0 && (!w->k || !w->v)) return KVQ_ERR_ARG;
  if (w->n > 0 && (!aligned16(w->k) || !aligned16(w->v))) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_ARG: return "KVQ_ERR_ARG: invalid argument";
    case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN: device pointer not 16-byte aligned";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: configuration not built";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: workspace missing or too small";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: kernel launch failed";
  }
  return "kvq: unknown status";
}

kvq_status kvq_quantize_pack(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                             int32_t H_kv, const uint16_t* k_src, const uint16_t* v_src,
                             int64_t src_head_stride, int64_t first_group, int64_t n_groups,
                             void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (B <= 0 || H_kv <= 0) return KVQ_ERR_ARG;
  if (first_group < 0 || n_groups < 0) return KVQ_ERR_ARG;
  const int64_t G = cfg->group;
  if (!groups_fit(cache, G, first_group + n_groups)) return KVQ_ERR_ARG;
  if (n_groups == 0) return KVQ_OK;
  if (!k_src || !v_src) return KVQ_ERR_ARG;
  if (src_head_stride < n_groups * G * kD) return KVQ_ERR_ARG;
  if (!aligned16(k_src) || !aligned16(v_src) || (src_head_stride * 2) % 16)
    return KVQ_ERR_ALIGN;
  const int64_t heads = (int64_t)B * H_kv;
  if (heads * n_groups > 0x7FFFFFFF) return KVQ_ERR_ARG;
  kvq::QuantArgs a{cache_args(cache), k_src,          v_src,        src_head_stride,
                   first_group,       n_groups,       (int32_t)heads, cfg->n_boost,
                   cfg->boost_score};
  return hip_status(kvq::launch_quantize(cfg->bits, vbits(cfg), cfg->group, a,
                                         static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_plan(const kvq_qcfg* cfg, int32_t B, int32_t H_q, int32_t H_kv,
                           int64_t n_quant_tokens, int32_t n_chunks_req, int32_t* n_chunks,
                           size_t* ws_bytes) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  if (B <= 0 || H_kv <= 0 || H_q <= 0 || H_q % H_kv) return KVQ_ERR_ARG;
  const int32_t gqa = H_q / H_kv;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_ERR_UNSUPPORTED;
  if (n_quant_tokens < 0 || n_quant_tokens % cfg->group || n_chunks_req < 0)
    return KVQ_ERR_ARG;
  const int64_t heads = (int64_t)B * H_kv;
  if (heads > 65535) return KVQ_ERR_ARG;  // one grid row per (batch, kv head)
  const bool mfma = kvq::mfma_decode_supported(same_bits(cfg), cfg->group, gqa, cfg->n_boost);
  const int32_t n = plan_chunks(mfma, cfg->bits, gqa, heads, n_quant_tokens / cfg->group, n_chunks_req);
  if (n_chunks) *n_chunks = n;
  if (ws_bytes) *ws_bytes = workspace_bytes(B, H_q, mfma ? n : n + 1);
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_qcfg* cfg, int32_t B, int32_t H_q, int32_t H_kv,
                                  int64_t n_quant_tokens, int32_t n_chunks_req) {
  size_t ws = 0;
  if (kvq_decode_plan(cfg, B, H_q, H_kv, n_quant_tokens, n_chunks_req, nullptr, &ws) != KVQ_OK)
    return 0;
  return ws;
}

}  // extern "C"

namespace {

// Validates a decode call and fills the launch arguments (shared by the
// one-call and the two-phase entry points).
kvq_status prepare_decode(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_q,
                          int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                          const kvq_window* sink, const kvq_window* res, float sm_scale,
                          int32_t n_chunks, void* workspace, size_t ws_bytes,
                          kvq::DecodeArgs* a) {
  int32_t nc = 0;
  size_t need = 0;
  kvq_status st = kvq_decode_plan(cfg, B, H_q, H_kv, n_quant_tokens, n_chunks, &nc, &need);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (!groups_fit(cache, cfg->group, n_quant_tokens / cfg->group)) return KVQ_ERR_ARG;
  if ((st = check_window(sink)) != KVQ_OK) return st;
  if ((st = check_window(res)) != KVQ_OK) return st;
  if (!q) return KVQ_ERR_ARG;
  if (!aligned16(q)) return KVQ_ERR_ALIGN;
  if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (!(sm_scale > 0.f)) sm_scale = 1.0f / sqrtf((float)kD);

  *a = kvq::DecodeArgs{};
  a->c = cache_args(cache);
  a->q = q;
  a->B = B;
  a->H_q = H_q;
  a->H_kv = H_kv;
  a->gqa = H_q / H_kv;
  a->n_boost = cfg->n_boost;
  a->n_groups = n_quant_tokens / cfg->group;
  a->n_chunks = nc;
  a->groups_per_chunk = nc > 0 ? (int32_t)((a->n_groups + nc - 1) / nc) : 0;
  if (sink && sink->n > 0) {
    a->k_sink = sink->k;
    a->v_sink = sink->v;
    a->n_sink = sink->n;
    a->sink_cap = sink->cap;
  }
  if (res && res->n > 0) {
    a->k_res = res->k;
    a->v_res = res->v;
    a->n_res = res->n;
    a->res_cap = res->cap;
  }
  a->qscale = sm_scale * 1.4426950408889634f;
  a->ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kvq::kCounterBytes);
  a->n_parts = kvq::decode_parts(same_bits(cfg), cfg->group, a->gqa, cfg->n_boost, nc,
                                 (int64_t)B * H_kv);
  a->counters = nullptr;
  a->append = 0;
  a->seq_quant = nullptr;
  a->seq_res = nullptr;
  a->status = static_cast<int32_t*>(workspace) + kvq::kStatusIndex;
  return KVQ_OK;
}

// The decode step with its merge: one launch where the kernel merges in
// place, else the split-K launch and the merge launch.
kvq_status decode_and_merge(const kvq_qcfg* cfg, kvq::DecodeArgs& a, void* workspace,
                            hipStream_t s) {
  if (kvq::fused_merge_supported(same_bits(cfg), cfg->group, a.gqa, cfg->n_boost, a.n_chunks,
                                 (int64_t)a.B * a.H_kv)) {
    a.counters = static_cast<int32_t*>(workspace);
    return hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s));
  }
  kvq_status st =
      hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s));
  if (st != KVQ_OK) return st;
  return hip_status(kvq::launch_merge(a, s));
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                int32_t H_q, int32_t H_kv, const uint16_t* q,
                                int64_t n_quant_tokens, const kvq_window* sink,
                                const kvq_window* res, float sm_scale, int32_t n_chunks,
                                void* workspace, size_t ws_bytes, float* out, void* stream) {
  kvq::DecodeArgs a;
  kvq_status st = prepare_decode(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                 sm_scale, n_chunks, workspace, ws_bytes, &a);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(out)) return KVQ_ERR_ALIGN;
  a.out = out;
  return decode_and_merge(cfg, a, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Validation of kvq_decode_step on a given workspace (the caller's, or the
// no-allocation entry point's scratch array): fills the launch arguments.
kvq_status prepare_step(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_q,
                        int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                        const kvq_window* sink, const kvq_window* res, float sm_scale,
                        int32_t n_chunks, void* workspace, size_t ws_bytes, float* out,
                        int32_t append, kvq::DecodeArgs* a) {
  kvq_status st = prepare_decode(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                 sm_scale, n_chunks, workspace, ws_bytes, a);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(out)) return KVQ_ERR_ALIGN;
  const int64_t G = cfg->group;
  if (append) {
    // the residual holds the full group that becomes group n_quant_tokens / G
    if (!res || res->n < G || !groups_fit(cache, G, n_quant_tokens / G + 1)) return KVQ_ERR_ARG;
    if ((int64_t)H_kv * B * 8 + (int64_t)B * H_q > 0x7FFFFFFF) return KVQ_ERR_ARG;
  }
  a->out = out;
  return KVQ_OK;
}

// The launches of a validated kvq_decode_step.
kvq_status launch_step(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_kv,
                       int64_t n_quant_tokens, const kvq_window* res, void* workspace,
                       int32_t append, kvq::DecodeArgs& a, void* stream) {
  kvq_status st;
  const int64_t G = cfg->group;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!append) return decode_and_merge(cfg, a, workspace, s);
  if (kvq::kitty_tail_append_supported(same_bits(cfg), cfg->group, a.gqa, cfg->n_boost,
                                       cfg->boost_score, a.n_chunks, (int64_t)B * H_kv)) {
    // one launch: the split-K kernel merges in place, then its blocks
    // quantize the appended group (Kitty key items, value items)
    a.append = 1;
    a.counters = static_cast<int32_t*>(workspace);
    return hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s));
  }
  if (kvq::split_append_supported(same_bits(cfg), cfg->group, a.gqa, cfg->n_boost, a.n_chunks) ||
      kvq::tail_append_supported(same_bits(cfg), cfg->group, a.gqa, cfg->n_boost)) {
    // the split-K launch also quantizes the appended group (2-bit: in its
    // consumer waves; 4-bit: in blocks after its decode grid); the merge runs
    // in the same launch (at most 8 parts) or in one launch after it
    a.append = 1;
    if (kvq::fused_merge_supported(same_bits(cfg), cfg->group, a.gqa, cfg->n_boost, a.n_chunks,
                                 (int64_t)a.B * a.H_kv)) {
      a.counters = static_cast<int32_t*>(workspace);
      return hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s));
    }
    if ((st = hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s))) !=
        KVQ_OK)
      return st;
    return hip_status(kvq::launch_merge(a, s));
  }
  if ((st = hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a, s))) !=
      KVQ_OK)
    return st;
  const int64_t heads = (int64_t)B * H_kv;
  const kvq::QuantArgs qa{cache_args(cache), res->k,         res->v,       (int64_t)res->cap * kD,
                          n_quant_tokens / G, 1,             (int32_t)heads, cfg->n_boost,
                          cfg->boost_score};
  return hip_status(kvq::launch_merge_append(cfg->bits, vbits(cfg), cfg->group, a, qa, s));
}

// ------------------------------------------------------------ no-allocation step
//
// The decode workspace of kvq_decode_step_noalloc: one array per GPU, in the
// library's code object, holding the counter bytes and the partial records.
// Its address on a device comes from hipGetSymbolAddress, taken once per
// device with that device current (the array's name in host code is a
// host-side stand-in, never a device address).
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address (resolved on the first call there).
kvq_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVQ_ERR_HIP;
  if (dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return KVQ_OK;
}

// Zeroes n int32 words (a kernel, not a memset, so a captured graph replays
// it as an ordinary kernel node).
__global__ void zero_words_kernel(int32_t* p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_step(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_q,
                           int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                           const kvq_window* sink, const kvq_window* res, float sm_scale,
                           int32_t n_chunks, void* workspace, size_t ws_bytes, float* out,
                           int32_t append, void* stream) {
  kvq::DecodeArgs a;
  const kvq_status st = prepare_step(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                     sm_scale, n_chunks, workspace, ws_bytes, out, append, &a);
  if (st != KVQ_OK) return st;
  return launch_step(cfg, cache, B, H_kv, n_quant_tokens, res, workspace, append, a, stream);
}

kvq_status kvq_decode_step_noalloc(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                   int32_t H_q, int32_t H_kv, const uint16_t* q,
                                   int64_t n_quant_tokens, const kvq_window* sink,
                                   const kvq_window* res, float sm_scale, int32_t n_chunks,
                                   float* out, int32_t append, void* stream) {
  // the workspace this call needs must fit the scratch array
  size_t need = 0;
  kvq_status st = kvq_decode_plan(cfg, B, H_q, H_kv, n_quant_tokens, n_chunks, nullptr, &need);
  if (st != KVQ_OK) return st;
  if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != KVQ_OK) return st;
  kvq::DecodeArgs a;
  if ((st = prepare_step(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res, sm_scale,
                         n_chunks, ws, KVQ_NOALLOC_SCRATCH_BYTES, out, append, &a)) != KVQ_OK)
    return st;
  // The array keeps the previous call's contents: zero the arrival counters
  // of this call's heads and the status words before the step.
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t heads = B * H_kv;   // <= 65535: checked by kvq_decode_plan above
  zero_words_kernel<<<(heads + 255) / 256, 256, 0, s>>>(static_cast<int32_t*>(ws), heads);
  zero_words_kernel<<<1, 64, 0, s>>>(static_cast<int32_t*>(ws) + kvq::kStatusIndex, 2);
  if ((st = hip_status(hipGetLastError())) != KVQ_OK) return st;
  return launch_step(cfg, cache, B, H_kv, n_quant_tokens, res, ws, append, a, stream);
}

kvq_status kvq_decode_partials(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                               int32_t H_q, int32_t H_kv, const uint16_t* q,
                               int64_t n_quant_tokens, const kvq_window* sink,
                               const kvq_window* res, float sm_scale, int32_t n_chunks,
                               void* workspace, size_t ws_bytes, int32_t* n_parts,
                               void* stream) {
  kvq::DecodeArgs a;
  kvq_status st = prepare_decode(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                 sm_scale, n_chunks, workspace, ws_bytes, &a);
  if (st != KVQ_OK) return st;
  if (!n_parts) return KVQ_ERR_ARG;
  *n_parts = a.n_parts;
  return hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a,
                                                static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attention_ragged(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                       int32_t H_q, int32_t H_kv, const uint16_t* q,
                                       int64_t n_quant_tokens, const kvq_window* sink,
                                       const kvq_window* res, const int32_t* seq_quant_tokens,
                                       const int32_t* seq_res_tokens, float sm_scale,
                                       int32_t n_chunks, void* workspace, size_t ws_bytes,
                                       float* out, void* stream) {
  kvq::DecodeArgs a;
  kvq_status st = prepare_decode(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                 sm_scale, n_chunks, workspace, ws_bytes, &a);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(out)) return KVQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(seq_quant_tokens) | reinterpret_cast<uintptr_t>(seq_res_tokens)) & 3u)
    return KVQ_ERR_ALIGN;
  a.out = out;
  a.seq_quant = seq_quant_tokens;
  a.seq_res = seq_res_tokens;
  return decode_and_merge(cfg, a, workspace, static_cast<hipStream_t>(stream));
}

kvq_status kvq_decode_partials_ragged(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B,
                                      int32_t H_q, int32_t H_kv, const uint16_t* q,
                                      int64_t n_quant_tokens, const kvq_window* sink,
                                      const kvq_window* res, const int32_t* seq_quant_tokens,
                                      const int32_t* seq_res_tokens, float sm_scale,
                                      int32_t n_chunks, void* workspace, size_t ws_bytes,
                                      int32_t* n_parts, void* stream) {
  kvq::DecodeArgs a;
  kvq_status st = prepare_decode(cfg, cache, B, H_q, H_kv, q, n_quant_tokens, sink, res,
                                 sm_scale, n_chunks, workspace, ws_bytes, &a);
  if (st != KVQ_OK) return st;
  if (!n_parts) return KVQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(seq_quant_tokens) | reinterpret_cast<uintptr_t>(seq_res_tokens)) & 3u)
    return KVQ_ERR_ALIGN;
  *n_parts = a.n_parts;
  a.seq_quant = seq_quant_tokens;
  a.seq_res = seq_res_tokens;
  return hip_status(kvq::launch_decode_partials(cfg->bits, vbits(cfg), cfg->group, a,
                                                static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_merge(int32_t B, int32_t H_q, int32_t n_parts, const float* workspace,
                            size_t ws_bytes, float* out, void* stream) {
  if (B <= 0 || H_q <= 0 || n_parts <= 0 || n_parts > kvq::kMaxParts) return KVQ_ERR_ARG;
  if ((int64_t)B * H_q > 0x7FFFFFFF) return KVQ_ERR_ARG;
  if (!workspace || ws_bytes < kvq::kCounterBytes + (size_t)B * H_q * n_parts * (kD + 2) * sizeof(float))
    return KVQ_ERR_WORKSPACE;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(workspace) || !aligned16(out)) return KVQ_ERR_ALIGN;
  kvq::DecodeArgs a{};
  a.B = B;
  a.H_q = H_q;
  a.n_parts = n_parts;
  a.ws = reinterpret_cast<float*>(
      const_cast<char*>(reinterpret_cast<const char*>(workspace)) + kvq::kCounterBytes);
  a.out = out;
  return hip_status(kvq::launch_merge(a, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_dequantize(const kvq_qcfg* cfg, const kvq_cache* cache, int32_t B, int32_t H_kv,
                          int64_t first_group, int64_t n_groups, float* k_out, float* v_out,
                          void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != KVQ_OK) return st;
  if (B <= 0 || H_kv <= 0 || first_group < 0 || n_groups < 0) return KVQ_ERR_ARG;
  if (!groups_fit(cache, cfg->group, first_group + n_groups)) return KVQ_ERR_ARG;
  if (n_groups == 0) return KVQ_OK;
  if (!k_out || !v_out) return KVQ_ERR_ARG;
  if (!aligned16(k_out) || !aligned16(v_out)) return KVQ_ERR_ALIGN;
  const int64_t heads = (int64_t)B * H_kv;
  if (heads * n_groups * cfg->group * kD / 256 > 0x7FFFFFFF) return KVQ_ERR_ARG;
  kvq::DequantArgs a{cache_args(cache), k_out, v_out, first_group, n_groups, (int32_t)heads,
                     cfg->n_boost};
  return hip_status(kvq::launch_dequantize(cfg->bits, vbits(cfg), cfg->group, a,
                                           static_cast<hipStream_t>(stream)));
}

kvq_status kvq_mx_decode_plan(int32_t B, int32_t H_q, int32_t H_kv, int64_t n_quant_tokens,
                              int32_t n_chunks_req, int32_t* n_chunks, size_t* ws_bytes) {
  if (B <= 0 || H_kv <= 0 || H_q <= 0 || H_q % H_kv) return KVQ_ERR_ARG;
  const int32_t gqa = H_q / H_kv;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8) return KVQ_ERR_UNSUPPORTED;
  if (n_quant_tokens < 0 || n_quant_tokens % 32 || n_chunks_req < 0) return KVQ_ERR_ARG;
  const int64_t heads = (int64_t)B * H_kv;
  if (heads > 65535) return KVQ_ERR_ARG;
  if (kvq::mx_mfma_supported(gqa, n_quant_tokens)) {
    // matrix-core kernel: chunks of 128-token groups, one resident block per
    // CU (the grid runs in one round), windows spread over the chunks
    const int64_t groups = n_quant_tokens / 128;
    int64_t n = n_chunks_req > 0 ? n_chunks_req : kvq::kCUs / heads;
    n = std::max<int64_t>(1, std::min<int64_t>({n, std::max<int64_t>(1, groups), kMaxChunks}));
    if (n_chunks) *n_chunks = (int32_t)n;
    if (ws_bytes) *ws_bytes = workspace_bytes(B, H_q, n);
    return KVQ_OK;
  }
  const int64_t blocks = n_quant_tokens / 32;
  int64_t n = n_chunks_req;
  // automatic: about 16 blocks per CU (the vector-ALU kernel is bound by
  // latency; 64 chunks per head ran the benchmark shape 1.7x faster than 8)
  if (n == 0) n = (4096 + heads - 1) / heads;
  n = std::max<int64_t>(1, std::min<int64_t>(n, std::max<int64_t>(1, blocks)));
  if (n > 65535) return KVQ_ERR_ARG;
  if (n_chunks) *n_chunks = (int32_t)n;
  if (ws_bytes) *ws_bytes = workspace_bytes(B, H_q, n + 1);
  return KVQ_OK;
}

kvq_status kvq_mx_decode_attention(const kvq_mx_cache* cache, int32_t B, int32_t H_q,
                                   int32_t H_kv, const uint16_t* q, int64_t n_quant_tokens,
                                   const kvq_window* sink, const kvq_window* res, float sm_scale,
                                   int32_t n_chunks_req, void* workspace, size_t ws_bytes,
                                   float* out, void* stream) {
  if (!cache || !cache->k_codes || !cache->k_scale || !cache->v_codes || !cache->v_scale)
    return KVQ_ERR_ARG;
  if (cache->t_cap <= 0 || cache->t_cap % 32 || n_quant_tokens > cache->t_cap) return KVQ_ERR_ARG;
  if (!aligned16(cache->k_codes) || !aligned16(cache->k_scale) || !aligned16(cache->v_codes) ||
      !aligned16(cache->v_scale))
    return KVQ_ERR_ALIGN;
  int32_t nc = 0;
  size_t need = 0;
  kvq_status st = kvq_mx_decode_plan(B, H_q, H_kv, n_quant_tokens, n_chunks_req, &nc, &need);
  if (st != KVQ_OK) return st;
  if ((st = check_window(sink)) != KVQ_OK || (st = check_window(res)) != KVQ_OK) return st;
  if (!q || !out) return KVQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (!(sm_scale > 0.f)) sm_scale = 1.0f / sqrtf((float)kD);
  kvq::DecodeArgs a{};
  a.q = q;
  a.B = B;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.gqa = H_q / H_kv;
  a.n_groups = n_quant_tokens / 32;
  a.n_chunks = nc;
  a.groups_per_chunk = (int32_t)((a.n_groups + nc - 1) / nc);
  if (sink && sink->n > 0) {
    a.k_sink = sink->k;
    a.v_sink = sink->v;
    a.n_sink = sink->n;
    a.sink_cap = sink->cap;
  }
  if (res && res->n > 0) {
    a.k_res = res->k;
    a.v_res = res->v;
    a.n_res = res->n;
    a.res_cap = res->cap;
  }
  a.qscale = sm_scale * 1.4426950408889634f;
  a.n_parts = nc + 1;
  a.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + kvq::kCounterBytes);
  a.status = static_cast<int32_t*>(workspace) + kvq::kStatusIndex;
  a.out = out;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kvq::mx_mfma_supported(a.gqa, n_quant_tokens)) {
    a.n_groups = n_quant_tokens / 128;
    a.groups_per_chunk = (int32_t)((a.n_groups + nc - 1) / nc);
    a.n_parts = nc;
    if (nc <= kvq::kFusedMergeParts) {   // one launch: the last block of a head merges
      a.counters = static_cast<int32_t*>(workspace);
      return hip_status(kvq::launch_decode_mx_mfma(*cache, a, s));
    }
    if ((st = hip_status(kvq::launch_decode_mx_mfma(*cache, a, s))) != KVQ_OK) return st;
    return hip_status(kvq::launch_merge(a, s));
  }
  if ((st = hip_status(kvq::launch_decode_mx(*cache, a, s))) != KVQ_OK) return st;
  return hip_status(kvq::launch_merge(a, s));
}

}  // extern "C"
