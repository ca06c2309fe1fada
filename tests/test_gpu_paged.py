"""GPU parity of the paged cache (one group per page, a page table per head):
quantize into a shuffled pool, decode through the table, append into a page,
all against the oracle over the same inputs in the contiguous layout (the
oracle knows no pages: the test gathers the pool into that layout by the
table, which is plain indexing).  A table entry outside the pool poisons only
its own head."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (TOL, assert_cache_equal, make_inputs, max_err, oracle_decode,
                         oracle_quantize, qcfg)
from test_gpu_parity import _w

pytestmark = pytest.mark.gpu

CASES = ["llama_2bit", "gqa8_2bit", "llama_4bit", "kitty_gqa4", "g32_8bit_gqa2", "k2v4", "kitty_mag"]


@pytest.fixture(scope="module")
def built():
    import bit_kv_cache_amd  # noqa: F401
    assert torch.cuda.is_available()
    return True


def _table(heads, n_groups, extra, seed):
    """A random injective page table [heads][n_groups] over a pool of
    heads * n_groups + extra pages."""
    n_pages = heads * n_groups + extra
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    return perm[: heads * n_groups].view(heads, n_groups).to(torch.int32), n_pages


def _gather(pool, table, n_groups):
    """The pool's pages in the contiguous layout ([heads][n_groups*G]...)."""
    import bit_kv_cache_amd as kvq
    cfg = pool.cfg
    G, fpi = cfg.group, 32 // cfg.vb
    idx = table[:, :n_groups].long().cpu()
    heads = idx.shape[0]
    n_pages = pool.t_cap // G

    def per_page(t, rows):   # [1][n_pages*rows][...] -> [n_pages][rows][...]
        return t.view(n_pages, rows, *t.shape[2:]).cpu()

    def take(t, rows):
        p = per_page(t, rows)
        return p[idx].reshape(heads, n_groups * rows, *p.shape[2:])

    f = dict(k_codes=take(pool.k_codes, G), k_scale=take(pool.k_scale, 1),
             k_min=take(pool.k_min, 1), v_codes=take(pool.v_codes, G // fpi),
             v_scale=take(pool.v_scale, G), v_min=take(pool.v_min, G),
             k_hi=take(pool.k_hi, G) if pool.k_hi is not None else None,
             k_bidx=take(pool.k_bidx, 1) if pool.k_bidx is not None else None)
    return kvq.Cache(cfg, n_groups * G, heads, **f)


@pytest.mark.parametrize("name", CASES)
def test_paged_quantize_decode_append(built, name):
    import bit_kv_cache_amd as kvq
    w = _w(name)
    w = synth.shrink(w, R=w.G)
    inp = make_inputs(w)
    n = len(inp["heads"])
    B = n // w.H_kv
    ng = w.T // w.G
    table, n_pages = _table(n, ng + 1, extra=7, seed=11)
    pool = kvq.Cache.pool(qcfg(w), n_pages, table.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    t_cap = w.T + w.G
    oc = oracle_quantize(w, inp, t_cap)
    torch.cuda.synchronize()
    assert_cache_equal(_gather(pool, table, ng), oc, tokens=w.T)

    # decode through the table: several chunk counts (4..8 take the one-launch
    # path for plain 2-bit codes)
    ref = oracle_decode(w, oc, inp, w.T)
    sink = kvq.window(inp["k_sink"], inp["v_sink"], w.S)
    res = kvq.window(inp["k_res"], inp["v_res"], w.R)
    q = inp["q"][:B].contiguous()
    for n_chunks in (0, 3, 4, 7):
        _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
        ws = kvq.decode_workspace(ws_bytes)
        out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
        kvq.kvq_decode_attention(qcfg(w), pool, B, w.H_q, w.H_kv, q, w.T, sink, res, out, ws,
                                 n_chunks=n_chunks)
        torch.cuda.synchronize()
        err = max_err(out, ref)
        assert err <= TOL, f"{name} n_chunks={n_chunks}: max-abs {err:.3g}"

    # one step with the append: the full residual group lands in the page the
    # table gives group ng
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, 4)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_step(qcfg(w), pool, B, w.H_q, w.H_kv, q, w.T, sink, res, out, ws, True,
                        n_chunks=4)
    oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]), ng, 1)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL
    assert_cache_equal(_gather(pool, table, ng + 1), oc, tokens=t_cap)

    # dequantize through the table equals the oracle's dequantized cache
    ko = torch.empty((n, t_cap, w.D), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    kvq.kvq_dequantize(qcfg(w), pool, 1, n, 0, ng + 1, ko, vo)
    kr, vr = oracle.dequantize(oc, 0, ng + 1)
    torch.cuda.synchronize()
    assert np.array_equal(ko.cpu().numpy().view(np.uint32), kr.view(np.uint32))
    assert np.array_equal(vo.cpu().numpy().view(np.uint32), vr.view(np.uint32))


@pytest.mark.bad_pages
@pytest.mark.parametrize("name", ["llama_2bit", "llama_4bit", "g32_8bit_gqa2"])
def test_paged_bad_entry_poisons_only_its_head(built, name):
    """A table entry outside the pool is never dereferenced: quantize skips the
    group, decode returns NaN for that head's query rows and the right
    result for every other head, and the workspace's status words count one
    poisoned part (the chunk holding the bad group) and no stalled block."""
    import bit_kv_cache_amd as kvq
    w = _w(name)
    inp = make_inputs(w)
    n = len(inp["heads"])
    B = n // w.H_kv
    ng = w.T // w.G
    table, n_pages = _table(n, ng, extra=3, seed=5)
    pool = kvq.Cache.pool(qcfg(w), n_pages, table.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    bad_head = 1
    for bad_page in (-1, n_pages, 1 << 30):
        t2 = table.clone()
        t2[bad_head, ng // 2] = bad_page
        pool2 = kvq.Cache.pool(qcfg(w), n_pages, t2.cuda())
        for f in kvq.Cache.FIELDS:
            setattr(pool2, f, getattr(pool, f))
        # quantize with the bad entry: writes nothing for that group, the rest
        # as before (re-quantizing the same inputs leaves the pool unchanged)
        before = {f: getattr(pool, f).clone() for f in ("k_codes", "k_scale", "v_codes")}
        kvq.kvq_quantize_pack(qcfg(w), pool2, 1, n, inp["k"], inp["v"], 0, ng)
        torch.cuda.synchronize()
        for f, t in before.items():
            assert torch.equal(getattr(pool, f), t), f
        for n_chunks in (0, 4):
            _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
            ws = kvq.decode_workspace(ws_bytes)
            out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
            kvq.kvq_decode_attention(qcfg(w), pool2, B, w.H_q, w.H_kv, inp["q"][:B].contiguous(),
                                     w.T, kvq.window(inp["k_sink"], inp["v_sink"], w.S),
                                     kvq.window(inp["k_res"], inp["v_res"], w.R), out, ws,
                                     n_chunks=n_chunks)
            torch.cuda.synchronize()
            assert kvq.workspace_status(ws) == (0, 1), (bad_page, n_chunks)
            o = out.view(n, w.gqa, w.D)
            assert torch.isnan(o[bad_head]).all(), (bad_page, n_chunks)
            good = [h for h in range(n) if h != bad_head]
            ref = oracle_decode(w, oracle_quantize(w, inp), inp, w.T).reshape(n, w.gqa, w.D)
            err = float(np.max(np.abs(o[good].cpu().numpy().astype(np.float64) - ref[good])))
            assert err <= TOL, (bad_page, n_chunks, err)


def _seq_inputs(inp, b, H_kv):
    """The inputs of sequence b alone (its kv heads and query rows)."""
    hs = slice(b * H_kv, (b + 1) * H_kv)
    out = {k: (v[hs] if torch.is_tensor(v) and k != "q" else v) for k, v in inp.items()}
    out["q"] = inp["q"][b:b + 1]
    out["heads"] = inp["heads"][hs]
    return out


@pytest.mark.parametrize("name", CASES)
@pytest.mark.parametrize("paged", [False, True])
def test_ragged_batch(built, name, paged):
    """Sequences of different lengths in one call: sequence b attends to its
    first seq_quant[b] cached tokens and seq_res[b] residual tokens; each
    matches the oracle run on that sequence alone.  One sequence has no
    cached tokens, one a length that is not a multiple of G (rounded down)."""
    import bit_kv_cache_amd as kvq
    w = synth.shrink(_w(name), B=3)
    inp = make_inputs(w)
    n = len(inp["heads"])
    ng = w.T // w.G
    cfg = qcfg(w)
    if paged:
        table, n_pages = _table(n, ng, extra=5, seed=23)
        cache = kvq.Cache.pool(cfg, n_pages, table.cuda())
    else:
        cache = kvq.Cache.empty(cfg, n, w.T)
    kvq.kvq_quantize_pack(cfg, cache, w.B, w.H_kv, inp["k"], inp["v"], 0, ng)
    seq_quant = [w.T, (ng // 2) * w.G + w.G // 3, 0]
    seq_res = [w.R, w.R // 3, max(1, w.R // 2)]
    sq = torch.tensor(seq_quant, dtype=torch.int32, device="cuda")
    sr = torch.tensor(seq_res, dtype=torch.int32, device="cuda")
    sink = kvq.window(inp["k_sink"], inp["v_sink"], w.S)
    res = kvq.window(inp["k_res"], inp["v_res"], w.R)
    refs = []
    for b in range(w.B):
        wb = synth.shrink(w, B=1)
        ib = _seq_inputs(inp, b, w.H_kv)
        nq = (seq_quant[b] // w.G) * w.G
        ocb = oracle_quantize(wb, ib, w.T + w.G)
        refs.append(oracle_decode(wb, ocb, ib, nq, n_res=seq_res[b]))
    for n_chunks in (0, 3, 4):
        _, ws_bytes = kvq.kvq_decode_plan(cfg, w.B, w.H_q, w.H_kv, w.T, n_chunks)
        ws = kvq.decode_workspace(ws_bytes)
        out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
        kvq.kvq_decode_attention_ragged(cfg, cache, w.B, w.H_q, w.H_kv, inp["q"].contiguous(), w.T,
                                        sink, res, sq, sr, out, ws, n_chunks=n_chunks)
        torch.cuda.synchronize()
        for b in range(w.B):
            err = max_err(out[b:b + 1], refs[b])
            assert err <= TOL, f"{name} paged={paged} n_chunks={n_chunks} seq {b}: {err:.3g}"



@pytest.mark.bad_pages
@pytest.mark.parametrize("name", ["llama_2bit", "gqa8_2bit", "llama_4bit", "kitty", "kitty_gqa4"])
def test_paged_bad_append_page_writes_nothing(built, name):
    """A table entry outside the pool for the group being appended: the step
    (4 chunks: one launch, the append inside it) and the quantize of that
    group alone write nothing for that head and nothing outside the other
    heads' pages for the group, the other heads' appended group is
    bit-exact, and the attention over the cached groups is the oracle's
    with no part poisoned (the decode never reads the appended group)."""
    import bit_kv_cache_amd as kvq
    from parity_util import FIELDS
    w = _w(name)
    w = synth.shrink(w, R=w.G)
    inp = make_inputs(w)
    n = len(inp["heads"])
    B = n // w.H_kv
    ng = w.T // w.G
    bad = n // 2
    table, n_pages = _table(n, ng + 1, extra=5, seed=17)
    t_bad = table.clone()
    t_bad[bad, ng] = n_pages + 3
    pool = kvq.Cache.pool(qcfg(w), n_pages, t_bad.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    torch.cuda.synchronize()
    names = [f for f in kvq.Cache.FIELDS if getattr(pool, f) is not None and f != "page_table"]
    before = {f: getattr(pool, f).clone() for f in names}
    oc = oracle_quantize(w, inp, w.T + w.G)
    oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]), ng, 1)
    ref = oracle_decode(w, oracle_quantize(w, inp), inp, w.T)
    written = {int(t_bad[h, ng]) for h in range(n) if h != bad}
    good = [h for h in range(n) if h != bad]

    def check():
        # the good heads' groups (appended one included) through the valid table
        g = _gather(pool, table, ng + 1)
        for gname, oname in FIELDS:
            gv, ov = getattr(g, gname), getattr(oc, oname)
            if gv is None:
                continue
            gh = gv.cpu().numpy().view(ov.dtype)
            assert np.array_equal(gh[good], ov[good]), gname
        # every page but the good heads' appended ones is as before
        for f in names:
            now, was = getattr(pool, f), before[f]
            rows = now.shape[1] // n_pages
            for p in range(n_pages):
                if p not in written:
                    assert torch.equal(now[0, p * rows:(p + 1) * rows],
                                       was[0, p * rows:(p + 1) * rows]), (f, p)

    # one step with the append
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, 4)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_step(qcfg(w), pool, B, w.H_q, w.H_kv, inp["q"][:B].contiguous(), w.T,
                        kvq.window(inp["k_sink"], inp["v_sink"], w.S),
                        kvq.window(inp["k_res"], inp["v_res"], w.R), out, ws, True, n_chunks=4)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL
    assert kvq.workspace_status(ws) == (0, 0)
    check()
    # the quantize of the appended group alone, from the restored pool
    for f in names:
        getattr(pool, f).copy_(before[f])
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k_res"], inp["v_res"], ng, 1)
    torch.cuda.synchronize()
    check()
