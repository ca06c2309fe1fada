"""kvq_decode_step_noalloc (the decode step on the library's per-GPU scratch
array, for callers that cannot allocate) against kvq_decode_step on a
workspace of its own: the same inputs through both, several calls in a row
on the one scratch array, each later call with a smaller input than the one
before, covering the one-launch path (in-launch merge: arrival counters in
the scratch array), the split-K + merge/append launches and a many-part
split.  Outputs within the 2e-3 attention bar of each other and of the
oracle, appended groups bit-exact."""

import pytest
import torch

import oracle
import synth
from parity_util import (TOL, assert_cache_equal, gpu_quantize, make_inputs, max_err,
                         oracle_decode, oracle_quantize, qcfg)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# (workload, chunks): each call's input smaller than the one before
CALLS = [
    (synth.shrink(W["long_t1m_2bit_splitk"], T=80 * 128), 64),        # 640 groups, 64 parts
    (synth.shrink(W["llama3_8b_t32k_2bit"], B=2, T=19 * 128), 4),    # 304 groups, one launch
    (synth.shrink(W["llama3_8b_t8k_b32_4bit"], B=1, T=6 * 128), 3),   # 48 groups, merge + append
    (synth.shrink(W["llama3_8b_t32k_2bit"], B=1, T=5 * 128), 7),      # 40 groups, one launch
]


@pytest.fixture(scope="module")
def built():
    import bit_kv_cache_amd  # noqa: F401
    assert torch.cuda.is_available()
    return True


def _step(kvq, w, inp, n_chunks, noalloc):
    t_cap = w.T + w.G
    cache = gpu_quantize(w, inp, t_cap)
    B = len(inp["heads"]) // w.H_kv
    out = torch.empty((B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    args = (qcfg(w), cache, B, w.H_q, w.H_kv, inp["q"][:B].contiguous(), w.T,
            kvq.window(inp["k_sink"], inp["v_sink"], w.S),
            kvq.window(inp["k_res"], inp["v_res"], w.R), out)
    if noalloc:
        kvq.kvq_decode_step_noalloc(*args, True, n_chunks=n_chunks)
    else:
        _, ws_bytes = kvq.kvq_decode_plan(qcfg(w), B, w.H_q, w.H_kv, w.T, n_chunks)
        kvq.kvq_decode_step(*args, kvq.decode_workspace(ws_bytes), True, n_chunks=n_chunks)
    torch.cuda.synchronize()
    return out, cache


def test_noalloc_step_equals_workspace_step(built):
    import bit_kv_cache_amd as kvq
    for i, (w0, n_chunks) in enumerate(CALLS):
        w = synth.shrink(w0, R=w0.G)
        inp = make_inputs(w)
        print(f"call {i}: B={w.B} H_q={w.H_q} T={w.T} bits={w.bits} chunks={n_chunks}", flush=True)
        out_n, cache_n = _step(kvq, w, inp, n_chunks, noalloc=True)
        out_w, cache_w = _step(kvq, w, inp, n_chunks, noalloc=False)
        assert torch.isfinite(out_n).all(), i
        err = (out_n - out_w).abs().max().item()
        assert err <= TOL, f"call {i}: no-alloc vs workspace step differ by {err:.3g}"
        t_cap = w.T + w.G
        for f in ("k_codes", "k_scale", "k_min", "v_codes", "v_scale", "v_min"):
            assert torch.equal(getattr(cache_n, f), getattr(cache_w, f)), (i, f)
        # and both against the oracle
        oc = oracle_quantize(w, inp, t_cap)
        ref = oracle_decode(w, oc, inp, w.T)
        oracle.quantize_pack(oc, synth.as_bits(inp["k_res"]), synth.as_bits(inp["v_res"]),
                             w.T // w.G, 1)
        assert max_err(out_n, ref) <= TOL, i
        assert_cache_equal(cache_n, oc, tokens=t_cap)
