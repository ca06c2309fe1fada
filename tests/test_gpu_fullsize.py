"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the library's automatic chunk plan, or the workload's
minimum chunk count), checked on sampled heads.

Every head of the full cache is quantized on the GPU and one decode step runs
over all of them, appending the full residual group into the cache (the
benchmark's step, kvq_decode_step).  The oracle regenerates the sampled heads' seeded
inputs and recomputes just those heads: their packed codes, scales, mins (and
Kitty high words / indices) must be bit-exact over every token slot, and their
query heads' attention outputs within max-abs 2e-3 of the oracle's fp64
attention over the same dequantized cache."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, assert_cache_equal, max_err, qcfg

pytestmark = pytest.mark.gpu

FULL = ["llama3_8b_t32k_2bit", "llama3_8b_t8k_b32_4bit", "kitty_t128k_h64_boost16",
        "long_t1m_2bit_splitk"]


def sampled_heads(w, n=3):
    """First, last and one seeded head in between."""
    rng = np.random.default_rng(w.seed)
    mid = int(rng.integers(1, max(2, w.heads - 1))) if w.heads > 2 else 0
    return sorted({0, w.heads - 1, mid})[:n]


def build_full(w, kvq):
    cfg = qcfg(w)
    t_cap = w.T + w.G
    cache = kvq.Cache.empty(cfg, w.heads, t_cap)
    hb = max(1, min(w.heads, (1 << 30) // (w.T * w.D * 4)))   # ~1 GiB of fp16 source per batch
    for h0 in range(0, w.heads, hb):
        n = min(hb, w.heads - h0)
        ks, vs = zip(*[synth.head_kv(w, h, "cuda") for h in range(h0, h0 + n)])
        k, v = torch.stack(ks), torch.stack(vs)
        kvq.kvq_quantize_pack(cfg, cache.heads_view(h0, n), 1, n, k, v, 0, w.T // w.G)
        del k, v, ks, vs
    wins = [synth.head_windows(w, h, "cuda") for h in range(w.heads)]
    win = [torch.stack([x[i] for x in wins]) for i in range(4)]
    torch.cuda.synchronize()
    return cfg, cache, win


@pytest.fixture(scope="module")
def built():
    import bit_kv_cache_amd  # noqa: F401  (fails loudly when the library is missing)
    assert torch.cuda.is_available()
    return True


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_heads(built, name):
    import bit_kv_cache_amd as kvq
    w = synth.WORKLOADS[name]
    print(f"full-size parity: {name} heads={w.heads} T={w.T}", flush=True)
    cfg, cache, (k_sink, v_sink, k_res, v_res) = build_full(w, kvq)
    q = synth.query(w, "cuda")

    # one decode step over every head, chunk plan as in the benchmark
    n_chunks, ws_bytes = kvq.kvq_decode_plan(cfg, w.B, w.H_q, w.H_kv, w.T, w.min_chunks)
    if w.min_chunks:
        assert n_chunks >= w.min_chunks
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    # the benchmark's step: decode + append of the full residual group (when
    # the window holds one) in one call
    append = w.R >= w.G
    kvq.kvq_decode_step(cfg, cache, w.B, w.H_q, w.H_kv, q, w.T, kvq.window(k_sink, v_sink, w.S),
                        kvq.window(k_res, v_res, w.R), out, ws, append, n_chunks=w.min_chunks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()

    # the oracle over the sampled heads, as one cache of len(hs) heads
    # (batch i = sampled head i, one kv head each; threads over heads)
    hs = sampled_heads(w)
    oc = oracle.empty_cache(w.bits, w.G, w.D, w.n_boost, w.T + w.G, len(hs))
    ks, vs = [], []
    for h in hs:
        k, v = synth.head_kv(w, h, "cuda")
        ks.append(synth.as_bits(k))
        vs.append(synth.as_bits(v))
        del k, v
    oracle.quantize_pack(oc, np.stack(ks), np.stack(vs), 0, w.T // w.G, n_threads=len(hs))
    del ks, vs
    sel = lambda t: synth.as_bits(t[hs]) if t is not None and t.shape[1] else None
    kS, vS, kR, vR = sel(k_sink), sel(v_sink), sel(k_res), sel(v_res)
    qh = synth.as_bits(q)
    qs = np.stack([qh[h // w.H_kv, (h % w.H_kv) * w.gqa:(h % w.H_kv + 1) * w.gqa] for h in hs])
    ref = oracle.decode_attention(oc, len(hs), w.gqa, 1, qs, w.T, k_sink=kS, v_sink=vS,
                                  n_sink=w.S, k_res=kR, v_res=vR, n_res=w.R, n_threads=len(hs))
    if append:
        oracle.quantize_pack(oc, kR, vR, w.T // w.G, 1, n_threads=len(hs))
    for i, h in enumerate(hs):
        b, hk = divmod(h, w.H_kv)
        err = max_err(out[b, hk * w.gqa:(hk + 1) * w.gqa], ref[i])
        print(f"  head {h}: max-abs {err:.3g}", flush=True)
        assert err <= TOL, f"{name} head {h}: max-abs {err:.3g}"
        one = oracle.empty_cache(w.bits, w.G, w.D, w.n_boost, w.T + w.G, 1)
        for f in ("k_words", "k_scale", "k_min", "k_hi", "k_bidx", "v_words", "v_scale",
                  "v_min"):
            if getattr(oc, f) is not None:
                setattr(one, f, getattr(oc, f)[i:i + 1])
        assert_cache_equal(cache.heads_view(h, 1), one, tokens=w.T + (w.G if append else 0))
