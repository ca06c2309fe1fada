"""GPU parity of the quantizer's guard and edge groups (KIVI page, Step 1:
scale = (max - min)/(2^bits - 1), codes divide by it; the guard for
max == min and for a range whose scale rounds to zero in fp16).

Key channels (per group of G tokens) and value tokens (per group of G
channels) are planted, on a fixed pattern, with:
  * constant groups (max == min: scale 0, codes 0, dequantized value = min);
  * groups of signed zeros (-0 < +0: min -0, max +0, scale 0);
  * ranges of one fp16 subnormal step (2^-24) whose scale underflows fp16 to
    zero at every code width, around zero and at the smallest normal value;
  * ranges that give fp16-subnormal scales (subnormal values of both signs,
    values just above the smallest normal);
  * values near +-65504, the fp16 maximum (their fp32 range exceeds fp16's).
Every quantize path of the library sees them: kvq_quantize_pack on a
contiguous and on a paged cache, and the streaming append inside
kvq_decode_step -- the one-launch step of the 2-bit kernel (4 and 7 chunks)
and the merge + quantize launch of the other kernels (Kitty, 4-bit, 8-bit,
G 32).  Codes, scales, mins, Kitty high words / indices and
dequantized values must equal the oracle bit for bit.

Attention over such a cache must stay within 2e-3 of the oracle.  Keys near
+-65504 sit in two channels whose query entries are scaled by 2^-12, so that
their logits stay O(1): an fp32 kernel cannot resolve logits of order 1e4
to 2e-3 (their rounding alone is of that size), while the fp64 oracle can.
Values near +-65504 are a separate case: every error term of the output
scales with the values' magnitude (the p.V operand's fixed-point digits,
2^-17 of the largest p_t * scale_t of a 32-token block; the fp32 rounding of the logits, which moves the weights of
values of that size; the fp32 accumulation), so that case is held to the
bar relative to the values' scale, 2e-3 * max(1, |v|max / 4), as the
scaled-input parity tests are (N(0,1) values reach |v| of about 4).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (TOL, assert_cache_equal, make_inputs, max_err, oracle_decode,
                         oracle_quantize, qcfg)
from test_gpu_paged import _gather, _table

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

CASES = {
    # one-launch step (split-K + append + merge) at 4 and 7 chunks
    "2bit_gqa4": synth.shrink(W["llama3_8b_t32k_2bit"], B=1, T=6 * 128),
    "2bit_gqa8": synth.shrink(W["llama3_8b_t32k_2bit"], B=1, H_q=64, T=5 * 128, S=3),
    # merge + quantize launch
    "4bit_gqa4": synth.shrink(W["llama3_8b_t8k_b32_4bit"], B=1, T=5 * 128),
    "kitty_gqa8": synth.shrink(W["kitty_t128k_h64_boost16"], B=1, T=5 * 128, S=5),
    "kitty_gqa4": synth.shrink(W["kitty_t128k_h64_boost16"], B=1, H_q=32, T=4 * 128, S=5),
    "8bit_gqa4": synth.shrink(W["llama3_8b_t8k_b32_4bit"], B=1, T=4 * 128, bits=8),
    "2bit_g32_gqa2": synth.shrink(W["llama3_8b_t32k_2bit"], B=1, H_q=16, G=32, T=24 * 32,
                                  R=32),
}

HUGE_KEY_CHANNELS = (5, 77)   # the only key channels that take values near 65504
QUERY_DAMP = 2.0 ** -12       # their query entries are scaled by this

TINY = 2.0 ** -24             # smallest fp16 subnormal
MIN_NORMAL = 2.0 ** -14


def _kind(i, j, h):
    """Edge kind of a group, from its coordinates (a fixed pattern that puts
    every kind in every head, group and channel range)."""
    return (i + 7 * j + 3 * h) % 12


def _fill(rng, n, kind, huge_ok):
    """n fp16 values (float64) of one group of the given kind; kinds 0..5 are
    N(0,1) (left as they are: None)."""
    if kind == 6:                                        # constant
        return np.full(n, np.float16(rng.standard_normal() * 3), np.float64)
    if kind == 7:                                        # signed zeros, both present
        z = np.where(rng.random(n) < 0.5, -0.0, 0.0)
        z[0], z[1] = -0.0, 0.0
        return z
    if kind == 8:                                        # range one subnormal step
        a = [0.0, MIN_NORMAL, -MIN_NORMAL - TINY, 3 * TINY][rng.integers(4)]
        x = a + TINY * rng.integers(0, 2, n)
        x[0], x[1] = a, a + TINY
        return x
    if kind == 9:                                        # subnormal values, both signs
        i = rng.integers(-900, 901, n)
        i[0], i[1] = -900, 900
        return i * TINY
    if kind == 10:                                       # just above the smallest normal
        i = rng.integers(0, 1024, n)
        i[0], i[1] = 0, rng.integers(1, 1024)
        return MIN_NORMAL + i * TINY
    if kind == 11 and huge_ok:                           # near the fp16 maximum
        x = np.array(rng.uniform(-65504, 65504, n), np.float16).astype(np.float64)
        x[0], x[1] = -65504.0, 65504.0
        return x
    return None


def _plant(k, v, G, seed, huge_keys, huge_values):
    """Plant edge groups into fp16 K and V ([heads][rows][D], rows a multiple
    of G) in place.  Keys per (head, group, channel), values per (head,
    token, channel group)."""
    rng = np.random.default_rng(seed)
    kn = k.cpu().numpy().astype(np.float64)
    vn = v.cpu().numpy().astype(np.float64)
    heads, rows, D = kn.shape
    for h in range(heads):
        for g in range(rows // G):
            for d in range(D):
                x = _fill(rng, G, _kind(d, g, h),
                          huge_keys and d in HUGE_KEY_CHANNELS)
                if x is not None:
                    kn[h, g * G:(g + 1) * G, d] = x
        for t in range(rows):
            for c in range(D // G):
                x = _fill(rng, G, _kind(t, c, h + 1), huge_values)
                if x is not None:
                    vn[h, t, c * G:(c + 1) * G] = x
    k.copy_(torch.from_numpy(kn.astype(np.float16)))
    v.copy_(torch.from_numpy(vn.astype(np.float16)))


def _edge_inputs(w, seed, huge_values=False):
    """Workload inputs with edge groups in the quantized region and in the
    residual window (whose first G rows the step appends)."""
    inp = make_inputs(w, "cpu")
    _plant(inp["k"], inp["v"], w.G, seed, True, huge_values)
    _plant(inp["k_res"], inp["v_res"], w.G, seed + 1, True, huge_values)
    q = inp["q"].float()
    q[..., list(HUGE_KEY_CHANNELS)] *= QUERY_DAMP
    inp["q"] = q.half()
    return {k: (t.cuda() if torch.is_tensor(t) else t) for k, t in inp.items()}


@pytest.fixture(scope="module")
def built():
    import bit_kv_cache_amd  # noqa: F401
    assert torch.cuda.is_available()
    return True


def _tol(w, oc, huge_values):
    if not huge_values:
        return TOL
    _, vv = oracle.dequantize(oc, 0, oc.t_cap // w.G)
    return TOL * max(1.0, float(np.abs(vv).max()) / 4.0)


def _check_plant(oc):
    """The planted kinds reach the quantizer: zero scales, subnormal scales,
    negative-zero minima (a guard against a pattern that plants nothing)."""
    s = np.concatenate([oc.k_scale.ravel(), oc.v_scale.ravel()])
    m = np.concatenate([oc.k_min.ravel(), oc.v_min.ravel()])
    assert np.count_nonzero(s == 0) > 50
    assert np.count_nonzero((s > 0) & (s < 0x0400)) > 50       # subnormal fp16 scales
    assert np.count_nonzero(m == 0x8000) > 10                  # -0 minima


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("huge_values", [False, True])
def test_edge_groups_quantize_contiguous_and_paged(built, name, huge_values):
    import bit_kv_cache_amd as kvq
    w = synth.shrink(CASES[name], R=CASES[name].G)
    inp = _edge_inputs(w, 900 + len(name), huge_values)
    n = len(inp["heads"])
    ng = w.T // w.G
    oc = oracle_quantize(w, inp)
    _check_plant(oc)
    # contiguous
    gc = kvq.Cache.empty(qcfg(w), n, w.T + w.G)
    kvq.kvq_quantize_pack(qcfg(w), gc, 1, n, inp["k"], inp["v"], 0, ng)
    torch.cuda.synchronize()
    assert_cache_equal(gc, oc, tokens=w.T)
    ko = torch.empty((n, w.T, w.D), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    kvq.kvq_dequantize(qcfg(w), gc, 1, n, 0, ng, ko, vo)
    kr, vr = oracle.dequantize(oc, 0, ng)
    assert np.array_equal(ko.cpu().numpy().view(np.uint32), kr[:, :w.T].view(np.uint32))
    assert np.array_equal(vo.cpu().numpy().view(np.uint32), vr[:, :w.T].view(np.uint32))
    # paged: a shuffled table over a pool with spare pages
    table, n_pages = _table(n, ng, extra=3, seed=31)
    pool = kvq.Cache.pool(qcfg(w), n_pages, table.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    torch.cuda.synchronize()
    assert_cache_equal(_gather(pool, table, ng), oc, tokens=w.T)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("huge_values", [False, True])
def test_edge_groups_decode_step_with_append(built, name, huge_values):
    """The step's append quantizes edge groups (in the split-K launch at 4
    and 7 chunks for plain 2-bit codes, in the merge's launch otherwise)
    bit-exactly; the attention over the edge cache matches the oracle."""
    import bit_kv_cache_amd as kvq
    w = synth.shrink(CASES[name], R=CASES[name].G)
    inp = _edge_inputs(w, 700 + len(name), huge_values)
    n = len(inp["heads"])
    B = n // w.H_kv
    t_cap = w.T + w.G
    oc = oracle_quantize(w, inp, t_cap)
    ref = oracle_decode(w, oc, inp, w.T)
    oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]),
                         w.T // w.G, 1)
    tol = _tol(w, oc, huge_values)
    sink = kvq.window(inp["k_sink"], inp["v_sink"], w.S)
    res = kvq.window(inp["k_res"], inp["v_res"], w.R)
    q = inp["q"][:B].contiguous()
    for n_chunks in (0, 3, 4, 7):
        gc = kvq.Cache.empty(qcfg(w), n, t_cap)
        kvq.kvq_quantize_pack(qcfg(w), gc, 1, n, inp["k"], inp["v"], 0, w.T // w.G)
        _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
        ws = kvq.decode_workspace(ws_bytes)
        out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
        kvq.kvq_decode_step(qcfg(w), gc, B, w.H_q, w.H_kv, q, w.T, sink, res, out, ws, True,
                            n_chunks=n_chunks)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"{name} n_chunks={n_chunks}"
        err = max_err(out, ref)
        assert err <= tol, f"{name} n_chunks={n_chunks}: max-abs {err:.3g} (tol {tol:.3g})"
        assert_cache_equal(gc, oc, tokens=t_cap)
    # the next step reads the appended edge group like any other
    _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, t_cap, 4)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention(qcfg(w), gc, B, w.H_q, w.H_kv, q, t_cap, sink, None, out, ws,
                             n_chunks=4)
    torch.cuda.synchronize()
    err = max_err(out, oracle_decode(w, oc, inp, t_cap, n_res=0))
    assert err <= tol, f"{name} after append: max-abs {err:.3g} (tol {tol:.3g})"


@pytest.mark.parametrize("name", ["2bit_gqa4", "4bit_gqa4", "kitty_gqa8"])
def test_edge_groups_paged_append(built, name):
    """The one-launch and merge-launch appends write edge groups into the page
    the table names, bit-exactly."""
    import bit_kv_cache_amd as kvq
    w = synth.shrink(CASES[name], R=CASES[name].G)
    inp = _edge_inputs(w, 500 + len(name))
    n = len(inp["heads"])
    B = n // w.H_kv
    ng = w.T // w.G
    table, n_pages = _table(n, ng + 1, extra=5, seed=37)
    pool = kvq.Cache.pool(qcfg(w), n_pages, table.cuda())
    kvq.kvq_quantize_pack(qcfg(w), pool, 1, n, inp["k"], inp["v"], 0, ng)
    t_cap = w.T + w.G
    oc = oracle_quantize(w, inp, t_cap)
    ref = oracle_decode(w, oc, inp, w.T)
    oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]), ng, 1)
    for n_chunks in (3, 4):
        _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
        ws = kvq.decode_workspace(ws_bytes)
        out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
        kvq.kvq_decode_step(qcfg(w), pool, B, w.H_q, w.H_kv, inp["q"][:B].contiguous(), w.T,
                            kvq.window(inp["k_sink"], inp["v_sink"], w.S),
                            kvq.window(inp["k_res"], inp["v_res"], w.R), out, ws, True,
                            n_chunks=n_chunks)
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL, f"{name} n_chunks={n_chunks}"
        assert_cache_equal(_gather(pool, table, ng + 1), oc, tokens=t_cap)
