"""GPU parity of the MXFP4 cache (32-value blocks, E8M0 scale, E2M1 values):
quantize + pack and dequantize through the C ABI against the CPU oracle on
the same seeded inputs, bit for bit, including blocks of zeros, fp16
subnormals, values near the fp16 maximum and exact rounding ties."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

D = 128


def _inputs(heads, n, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((heads, n, D)).astype(np.float32)
    k[:, :, 3] *= 40.0                                   # an outlier channel
    k[:, 5, :] = 0.0                                     # a token of zeros: key blocks of 0
    k[:, 9, 64:96] *= 2.0 ** -20                         # fp16 subnormals
    k[:, 11, :32] = rng.choice([-1, 1], 32) * 60000.0    # near the fp16 maximum
    # exact ties: a block whose largest magnitude is 4 * 2^E and the rest midpoints
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.0])
    k[:, 13, 32:64] = np.resize(np.concatenate([[4.0], mids]), 32) * 2.0 ** -3
    v = (rng.standard_normal((heads, n, D)) * rng.uniform(0.05, 20.0, (1, 1, D))).astype(np.float32)
    v[:, 32:64, 7] = 0.0                                 # a value block of zeros
    v[:, 64:96, 8] = np.resize(np.concatenate([[6.0], -mids]), 32) * 2.0 ** 2
    return k.astype(np.float16), v.astype(np.float16)


def _compare(gc, oc, t_hi):
    assert np.array_equal(gc.k_codes.cpu().numpy().view(np.uint32)[:, :t_hi], oc.k_words[:, :t_hi])
    assert np.array_equal(gc.k_scale.cpu().numpy()[:, :t_hi], oc.k_scale[:, :t_hi])
    assert np.array_equal(gc.v_codes.cpu().numpy().view(np.uint32)[:, : t_hi // 8],
                          oc.v_words[:, : t_hi // 8])
    assert np.array_equal(gc.v_scale.cpu().numpy()[:, : t_hi // 32], oc.v_scale[:, : t_hi // 32])


@pytest.mark.parametrize("B,H_kv,n", [(1, 2, 256), (2, 3, 96)])
def test_mx_quantize_append_dequantize_bit_exact(B, H_kv, n):
    import bit_kv_cache_amd as kvq
    heads = B * H_kv
    t_cap = n + 64
    k, v = _inputs(heads, n + 32, seed=31 + n)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    gc = kvq.MxCache.empty(heads, t_cap)
    kvq.kvq_mx_quantize_pack(gc, B, H_kv, kt[:, :n], vt[:, :n], 0, n)
    # the next 32 tokens appended as their own call
    kvq.kvq_mx_quantize_pack(gc, B, H_kv, kt[:, n:], vt[:, n:], n, 32)
    oc = oracle.mx_empty_cache(D, t_cap, heads)
    oracle.mx_quantize_pack(oc, k.view(np.uint16)[:, :n], v.view(np.uint16)[:, :n], 0, n)
    oracle.mx_quantize_pack(oc, k.view(np.uint16)[:, n:], v.view(np.uint16)[:, n:], n, 32)
    torch.cuda.synchronize()
    _compare(gc, oc, n + 32)
    # slots past the appended block stay untouched
    assert int(gc.k_codes[:, n + 32:].abs().sum()) == 0 and int(gc.k_scale[:, n + 32:].sum()) == 0
    ko = torch.empty((heads, n + 32, D), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    kvq.kvq_mx_dequantize(gc, B, H_kv, 0, n + 32, ko, vo)
    kr, vr = oracle.mx_dequantize(oc, 0, n + 32)
    torch.cuda.synchronize()
    assert np.array_equal(ko.cpu().numpy().view(np.uint32), kr.view(np.uint32))
    assert np.array_equal(vo.cpu().numpy().view(np.uint32), vr.view(np.uint32))


# (B, H_q, H_kv, T, S, R): GQA 4 and 8 with whole 128-token groups take the
# block-scaled matrix-core kernel (one launch up to 8 parts per head, a merge
# launch past that); GQA 1 and 2 and token counts with a 32-token tail take
# the vector-ALU kernel.
MX_CASES = [(1, 32, 8, 512, 5, 40), (2, 16, 2, 224, 0, 17), (1, 8, 8, 96, 3, 1),
            (1, 32, 8, 0, 4, 9), (2, 16, 2, 640, 3, 33), (1, 32, 8, 2048, 0, 128),
            (3, 32, 4, 1152, 7, 64), (1, 64, 8, 896, 2, 5), (1, 16, 8, 256, 0, 3)]


@pytest.mark.parametrize("edges", [False, True])
@pytest.mark.parametrize("B,H_q,H_kv,T,S,R", MX_CASES)
def test_mx_decode_matches_oracle(B, H_q, H_kv, T, S, R, edges):
    """Decode over the MXFP4 cache (plus fp16 sink and residual windows) at
    several chunk counts: max-abs within 2e-3 of the oracle's fp64 attention
    over the same dequantized cache.  With edges, the cache also holds blocks
    of zeros (E8M0 byte 0), fp16 subnormals and exact E2M1 ties."""
    import bit_kv_cache_amd as kvq
    from parity_util import TOL, max_err
    heads = B * H_kv
    rng = np.random.default_rng(41 + T + H_q)
    k = rng.standard_normal((heads, max(T, 32), D)).astype(np.float32)
    k[:, :, 3] *= 10.0
    v = rng.standard_normal((heads, max(T, 32), D)).astype(np.float32)
    if edges and T >= 128:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.0])
        k[:, 5, :] = 0.0                                  # a token of zero key blocks
        k[:, 9, 64:96] *= 2.0 ** -20                      # fp16 subnormals
        k[:, 13, 32:64] = np.resize(np.concatenate([[4.0], mids]), 32) * 2.0 ** -3
        v[:, 32:64, 7] = 0.0                              # a value block of zeros
        v[:, 64:96, 8] = np.resize(np.concatenate([[6.0], -mids]), 32) * 2.0 ** 2
        v[:, 96:128, 20:40] *= 2.0 ** -18                 # value subnormals
    k, v = k.astype(np.float16), v.astype(np.float16)
    ks = rng.standard_normal((heads, max(S, 1), D)).astype(np.float16)
    vs = rng.standard_normal((heads, max(S, 1), D)).astype(np.float16)
    kr = rng.standard_normal((heads, R + 3, D)).astype(np.float16)
    vr = rng.standard_normal((heads, R + 3, D)).astype(np.float16)
    q = rng.standard_normal((B, H_q, D)).astype(np.float16)
    t_cap = max(T, 32) + 32
    gc = kvq.MxCache.empty(heads, t_cap)
    oc = oracle.mx_empty_cache(D, t_cap, heads)
    if T:
        kvq.kvq_mx_quantize_pack(gc, B, H_kv, torch.from_numpy(k).cuda(),
                                 torch.from_numpy(v).cuda(), 0, T)
        oracle.mx_quantize_pack(oc, k.view(np.uint16), v.view(np.uint16), 0, T)
    dev = lambda a: torch.from_numpy(a).cuda()
    ks_d, vs_d, kr_d, vr_d, q_d = dev(ks), dev(vs), dev(kr), dev(vr), dev(q)
    ref = oracle.mx_decode_attention(oc, B, H_q, H_kv, q.view(np.uint16), T,
                                     k_sink=ks.view(np.uint16) if S else None,
                                     v_sink=vs.view(np.uint16) if S else None, n_sink=S,
                                     k_res=kr.view(np.uint16), v_res=vr.view(np.uint16), n_res=R)
    for n_chunks in sorted({0, 1, 3, 7, 9, max(1, T // 128), max(1, T // 32)}):
        _, ws_bytes = kvq.kvq_mx_decode_plan(B, H_q, H_kv, T, n_chunks)
        ws = kvq.decode_workspace(ws_bytes)
        out = torch.empty((B, H_q, D), dtype=torch.float32, device="cuda")
        kvq.kvq_mx_decode_attention(gc, B, H_q, H_kv, q_d, T, kvq.window(ks_d, vs_d, S),
                                    kvq.window(kr_d, vr_d, R), out, ws, n_chunks=n_chunks)
        torch.cuda.synchronize()
        err = max_err(out, ref)
        assert err <= TOL, f"n_chunks={n_chunks}: max-abs {err:.3g}"
        # the in-launch merge leaves the arrival counters zero
        assert int(ws[: kvq.KVQ_WS_STATUS // 4].view(torch.int32).abs().sum().item()) == 0
