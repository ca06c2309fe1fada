"""GPU parity of the 2-bit kernel's one-chunk-per-wave geometry.

A step of many chunks per head (plain 2-bit codes at GQA 4, 4 or more
blocks' worth of chunks per head, enough chunks to fill every CU in one
round) runs with blocks of one loader and 8 consumer waves, each consumer
taking one whole chunk; the block merges its 8 chunks' softmax states into
one part, and with at most 32 such parts per head the last block of the
head merges them in the same launch.  These cases take that path (256
chunks over 8 kv heads, or 128 over 16) and check it against the oracle:
every chunk full; chunks of two groups with the last 106 chunks empty (so
a block holds both full and empty chunks); three groups with one partial
chunk; ragged sequence lengths, contiguous and paged; a bad page-table entry
(its block's part is poisoned and counted once); the step with the append,
whose group must land bit-exact; and the two phases apart (32 parts, then
the merge launch)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (TOL, assert_cache_equal, gpu_quantize, make_inputs, max_err,
                         oracle_decode, oracle_quantize, qcfg)
from test_gpu_paged import _gather, _seq_inputs, _table

pytestmark = pytest.mark.gpu

BASE = synth.WORKLOADS["long_t1m_2bit_splitk"]   # B 1, 32 query heads over 8 kv heads


def _shape(n_groups, **kw):
    return synth.shrink(BASE, T=n_groups * BASE.G, **kw)


@pytest.fixture(scope="module")
def built():
    import bit_kv_cache_amd  # noqa: F401  (fails loudly when the library is missing)
    assert torch.cuda.is_available()
    return True


def _decode(w, cache, inp, n_chunks, B=None):
    import bit_kv_cache_amd as kvq
    B = B or len(inp["heads"]) // w.H_kv
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention(qcfg(w), cache, B, w.H_q, w.H_kv, inp["q"][:B].contiguous(), w.T,
                             kvq.window(inp["k_sink"], inp["v_sink"], w.S),
                             kvq.window(inp["k_res"], inp["v_res"], w.R), out, ws,
                             n_chunks=n_chunks)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("n_groups,S", [(256, 0), (300, 5), (700, 0)])
def test_chunk_per_wave_decode(built, n_groups, S):
    import bit_kv_cache_amd as kvq
    w = _shape(n_groups, S=S)
    inp = make_inputs(w)
    gc = gpu_quantize(w, inp)
    ref = oracle_decode(w, oracle_quantize(w, inp), inp, w.T)
    out, ws = _decode(w, gc, inp, 256)
    err = max_err(out, ref)
    assert err <= TOL, f"{n_groups} groups: max-abs {err:.3g}"
    assert kvq.workspace_status(ws) == (0, 0)


def test_chunk_per_wave_step_with_append(built):
    """kvq_decode_step at 256 chunks: one launch (one chunk per wave, 32
    parts of 8 chunks merged in place) that also quantizes the full residual
    group."""
    import bit_kv_cache_amd as kvq
    w = _shape(300)
    inp = make_inputs(w)
    t_cap = w.T + w.G
    oc = oracle_quantize(w, inp, t_cap)
    ref = oracle_decode(w, oc, inp, w.T)
    oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]),
                         w.T // w.G, 1)
    gc = gpu_quantize(w, inp, t_cap)
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), w.B, w.H_q, w.H_kv, w.T, 256)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_step(qcfg(w), gc, w.B, w.H_q, w.H_kv, inp["q"].contiguous(), w.T,
                        kvq.window(inp["k_sink"], inp["v_sink"], w.S),
                        kvq.window(inp["k_res"], inp["v_res"], w.R), out, ws, True,
                        n_chunks=256)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL
    assert kvq.workspace_status(ws) == (0, 0)
    assert_cache_equal(gc, oc, tokens=t_cap)


@pytest.mark.parametrize("paged", [False, True])
def test_chunk_per_wave_ragged(built, paged):
    """Two sequences (16 kv heads, 128 chunks): the second attends to a
    length that ends inside a chunk and a shorter residual window."""
    import bit_kv_cache_amd as kvq
    w = _shape(300, B=2)
    inp = make_inputs(w)
    n = len(inp["heads"])
    ng = w.T // w.G
    cfg = qcfg(w)
    if paged:
        table, n_pages = _table(n, ng, extra=5, seed=31)
        cache = kvq.Cache.pool(cfg, n_pages, table.cuda())
    else:
        cache = kvq.Cache.empty(cfg, n, w.T)
    kvq.kvq_quantize_pack(cfg, cache, w.B, w.H_kv, inp["k"], inp["v"], 0, ng)
    seq_quant = [w.T, 133 * w.G + 50]
    seq_res = [w.R, 40]
    refs = []
    for b in range(w.B):
        wb = synth.shrink(w, B=1)
        ib = _seq_inputs(inp, b, w.H_kv)
        nq = (seq_quant[b] // w.G) * w.G
        refs.append(oracle_decode(wb, oracle_quantize(wb, ib, w.T + w.G), ib, nq,
                                  n_res=seq_res[b]))
    _, ws_bytes = kvq.kvq_decode_plan(cfg, w.B, w.H_q, w.H_kv, w.T, 128)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention_ragged(
        cfg, cache, w.B, w.H_q, w.H_kv, inp["q"].contiguous(), w.T,
        kvq.window(inp["k_sink"], inp["v_sink"], w.S), kvq.window(inp["k_res"], inp["v_res"], w.R),
        torch.tensor(seq_quant, dtype=torch.int32, device="cuda"),
        torch.tensor(seq_res, dtype=torch.int32, device="cuda"), out, ws, n_chunks=128)
    torch.cuda.synchronize()
    for b in range(w.B):
        err = max_err(out[b:b + 1], refs[b])
        assert err <= TOL, f"paged={paged} seq {b}: {err:.3g}"
    assert kvq.workspace_status(ws) == (0, 0)


@pytest.mark.bad_pages
def test_chunk_per_wave_bad_page_poisons_its_chunk(built):
    """A table entry outside the pool poisons the part (block of 8 chunks)
    holding it (NaN for that head, counted once) and nothing else."""
    import bit_kv_cache_amd as kvq
    w = _shape(256)
    inp = make_inputs(w)
    n = len(inp["heads"])
    ng = w.T // w.G
    table, n_pages = _table(n, ng, extra=3, seed=7)
    pool = kvq.Cache.pool(qcfg(w), n_pages, table.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    bad_head = 3
    t2 = table.clone()
    t2[bad_head, 100] = n_pages + 2
    pool2 = kvq.Cache.pool(qcfg(w), n_pages, t2.cuda())
    for f in kvq.Cache.FIELDS:
        setattr(pool2, f, getattr(pool, f))
    out, ws = _decode(w, pool2, inp, 256)
    assert kvq.workspace_status(ws) == (0, 1)
    o = out.view(n, w.gqa, w.D)
    assert torch.isnan(o[bad_head]).all()
    good = [h for h in range(n) if h != bad_head]
    oc = oracle_quantize(w, inp)
    torch.cuda.synchronize()
    assert_cache_equal(_gather(pool, table, ng), oc, tokens=w.T)
    ref = oracle_decode(w, oc, inp, w.T).reshape(n, w.gqa, w.D)
    err = float(np.max(np.abs(o[good].cpu().numpy().astype(np.float64) - ref[good])))
    assert err <= TOL, err


def test_chunk_per_wave_partials_then_merge(built):
    """kvq_decode_partials at 256 chunks gives 32 parts per (batch, query
    head), each the merged state of 8 chunks; kvq_decode_merge over them
    equals the one-launch call and the oracle."""
    import bit_kv_cache_amd as kvq
    w = _shape(300)
    inp = make_inputs(w)
    gc = gpu_quantize(w, inp)
    ref = oracle_decode(w, oracle_quantize(w, inp), inp, w.T)
    one, ws1 = _decode(w, gc, inp, 256)
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), w.B, w.H_q, w.H_kv, w.T, 256)
    ws = kvq.decode_workspace(ws_bytes)
    sink = kvq.window(inp["k_sink"], inp["v_sink"], w.S)
    res = kvq.window(inp["k_res"], inp["v_res"], w.R)
    n_parts = kvq.kvq_decode_partials(qcfg(w), gc, w.B, w.H_q, w.H_kv, inp["q"].contiguous(),
                                      w.T, sink, res, ws, n_chunks=256)
    assert n_parts == 256 // 8
    out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_merge(w.B, w.H_q, n_parts, ws, out)
    torch.cuda.synchronize()
    assert kvq.workspace_status(ws) == (0, 0) and kvq.workspace_status(ws1) == (0, 0)
    assert max_err(out, ref) <= TOL
    assert float((out - one).abs().max()) <= 1e-4
