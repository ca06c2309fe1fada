"""Helpers of the GPU parity tests: build seeded inputs, run the HIP path
through the C ABI, run the oracle on host copies of the same inputs, compare.

Only inputs flow from here to the oracle; nothing the HIP path computes is
ever handed to the oracle."""

from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import synth

TOL = 2e-3  # max-abs attention error vs the fp64 oracle


def qcfg(w):
    import bit_kv_cache_amd as kvq
    return kvq.QCfg(bits=w.bits, group=w.G, head_dim=w.D, n_boost=w.n_boost, v_bits=w.v_bits,
                    boost_score=w.boost_score)


def make_inputs(w, device="cuda", heads=None):
    """Source K/V of the quantized region, windows and q for the given heads
    (default all), stacked ``[n_heads][rows][D]`` fp16 on ``device``."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    ks, vs, kS, vS, kR, vR = [], [], [], [], [], []
    for h in heads:
        k, v = synth.head_kv(w, h, device)
        a, b, c, d = synth.head_windows(w, h, device)
        ks.append(k), vs.append(v), kS.append(a), vS.append(b), kR.append(c), vR.append(d)
    st = lambda xs: torch.stack(xs) if xs else None
    return dict(k=st(ks), v=st(vs), k_sink=st(kS), v_sink=st(vS), k_res=st(kR), v_res=st(vR),
                q=synth.query(w, device), heads=heads)


def gpu_quantize(w, inp, t_cap=None, stream=None):
    import bit_kv_cache_amd as kvq
    cfg = qcfg(w)
    n = len(inp["heads"])
    t_cap = t_cap or (w.T + max(w.R, w.G))
    cache = kvq.Cache.empty(cfg, n, t_cap)
    if w.T:
        kvq.kvq_quantize_pack(cfg, cache, 1, n, inp["k"], inp["v"], 0, w.T // w.G, stream=stream)
    return cache


def oracle_quantize(w, inp, t_cap=None):
    t_cap = t_cap or (w.T + max(w.R, w.G))
    n = len(inp["heads"])
    c = oracle.empty_cache(w.bits, w.G, w.D, w.n_boost, t_cap, n, v_bits=w.v_bits,
                           score=w.boost_score)
    if w.T:
        oracle.quantize_pack(c, synth.as_bits(inp["k"]), synth.as_bits(inp["v"]), 0, w.T // w.G)
    return c


FIELDS = [("k_codes", "k_words"), ("k_scale", "k_scale"), ("k_min", "k_min"),
          ("k_hi", "k_hi"), ("k_bidx", "k_bidx"), ("v_codes", "v_words"),
          ("v_scale", "v_scale"), ("v_min", "v_min")]


def assert_cache_equal(gc, oc, tokens=None):
    """Bit-exact comparison of every cache array (optionally only the first
    ``tokens`` token slots)."""
    G, v_fpi = oc.group, oc.v_fpi
    for gname, oname in FIELDS:
        g, o = getattr(gc, gname), getattr(oc, oname)
        if g is None or o is None:
            assert g is None and o is None, gname
            continue
        gh = g.cpu().numpy().view(o.dtype)
        if tokens is not None:
            rows = {"k_codes": tokens, "k_hi": tokens, "k_scale": tokens // G,
                    "k_min": tokens // G, "k_bidx": tokens // G, "v_codes": tokens // v_fpi,
                    "v_scale": tokens, "v_min": tokens}[gname]
            gh, o = gh[:, :rows], o[:, :rows]
        bad = np.argwhere(gh != o)
        assert bad.size == 0, f"{gname}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


def gpu_decode(w, cache, inp, n_quant, n_chunks=0, n_res=None, n_sink=None, stream=None):
    import bit_kv_cache_amd as kvq
    cfg = qcfg(w)
    n = len(inp["heads"])
    B = n // w.H_kv
    n_res = w.R if n_res is None else n_res
    n_sink = w.S if n_sink is None else n_sink
    _, ws_bytes = kvq.kvq_decode_plan(cfg, B, w.H_q, w.H_kv, n_quant, n_chunks)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    q = inp["q"][:B].contiguous()
    kvq.kvq_decode_attention(cfg, cache, B, w.H_q, w.H_kv, q, n_quant,
                             kvq.window(inp["k_sink"], inp["v_sink"], n_sink),
                             kvq.window(inp["k_res"], inp["v_res"], n_res), out, ws,
                             n_chunks=n_chunks, stream=stream)
    return out


def oracle_decode(w, oc, inp, n_quant, n_res=None, n_sink=None):
    n = len(inp["heads"])
    B = n // w.H_kv
    n_res = w.R if n_res is None else n_res
    n_sink = w.S if n_sink is None else n_sink
    bits = lambda t: None if t is None else synth.as_bits(t)
    return oracle.decode_attention(
        oc, B, w.H_q, w.H_kv, synth.as_bits(inp["q"][:B]), n_quant,
        k_sink=bits(inp["k_sink"]) if n_sink else None,
        v_sink=bits(inp["v_sink"]) if n_sink else None, n_sink=n_sink,
        k_res=bits(inp["k_res"]) if n_res else None,
        v_res=bits(inp["v_res"]) if n_res else None, n_res=n_res)


# (test id, max-abs error) of every comparison made through max_err, printed
# at the end of the session (tests/conftest.py) so that the margins below the
# bar are on record even in a quiet run
ERRORS = []


def max_err(gpu_out, ref):
    err = float(np.max(np.abs(gpu_out.cpu().numpy().astype(np.float64) - ref)))
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    ERRORS.append((test, err))
    return err
