"""Pins of the MXFP4 part of the oracle (BitDecoding page, native
low-precision formats mxfp4 / nvfp4; the format is the OCP microscaling one:
32-value blocks, an E8M0 power-of-two scale, E2M1 values).  Each test checks
the oracle against the format's definition written out here, hand-worked
cases, or an independent brute force in numpy.  CPU only."""

import math

import numpy as np
import pytest

import oracle


def e2m1_from_bits(code):
    """E2M1 from its fields: sign bit 3, exponent bits 2..1 (bias 1; 0 is
    subnormal), mantissa bit 0."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return -mag if s else mag


def test_e2m1_values_follow_the_field_definition():
    for c in range(16):
        assert oracle.fp4_value(c) == e2m1_from_bits(c)
        assert math.copysign(1, oracle.fp4_value(c)) == (-1 if c & 8 else 1)
    assert sorted({abs(e2m1_from_bits(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("v,code", [
    (0.0, 0), (-0.0, 8), (0.5, 1), (6.0, 7), (-6.0, 15),
    # ties go to the even mantissa bit
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (-5.0, 14),
    # just off a tie
    (0.2500001, 1), (4.999999, 6), (5.000001, 7),
    # past the largest magnitude: saturate
    (6.9, 7), (7.99, 7), (1e9, 7), (-1e9, 15),
])
def test_e2m1_rounding_hand_cases(v, code):
    assert oracle.fp4_encode(v) == code


def test_e2m1_rounding_is_nearest_brute_force():
    rng = np.random.default_rng(21)
    grid = np.array([e2m1_from_bits(c) for c in range(16)])
    for v in rng.uniform(-8.5, 8.5, 4000):
        c = oracle.fp4_encode(v)
        assert abs(v - grid[c]) == np.min(np.abs(v - grid)), v
        assert (c >> 3) == (1 if v < 0 else 0)


def _blk(*vals):
    x = np.zeros(32, np.float16)
    x[: len(vals)] = vals
    return x.view(np.uint16)


@pytest.mark.parametrize("vals,E", [
    ((6.0,), 0), ((4.0, -1.0), 0), ((7.99,), 0), ((1.0,), -2), ((-1.0, 0.5), -2),
    ((0.375,), -4), ((65504.0,), 13), ((2.0 ** -24,), -26), ((0.0,), -127),
])
def test_shared_exponent_hand_cases(vals, E):
    """E = floor(log2(max |x|)) - 2; a block of zeros gives -127."""
    assert oracle.mx_exponent(_blk(*vals)) == E


def test_representable_block_is_exact():
    """Values k 2^E with k on the E2M1 grid and max |k| in {4, 6} come back
    exactly."""
    rng = np.random.default_rng(22)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for E in (-6, -2, 0, 3):
        for top in (4.0, 6.0):
            k = rng.choice(grid[grid <= top], 32) * rng.choice([-1, 1], 32)
            k[rng.integers(32)] = top
            x = (k * 2.0 ** E).astype(np.float16)
            assert oracle.mx_exponent(x.view(np.uint16)) == E
            for xi in x:
                code = oracle.fp4_encode(float(xi) / 2.0 ** E)
                assert oracle.mx_dequant(code, E + 127) == float(xi)


def _mx_numpy(blocks):
    """Independent brute force: [n][32] float16 -> (E per block, x_hat)."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    xf = blocks.astype(np.float64)
    amax = np.abs(xf).max(1)
    E = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, -127).astype(int)
    y = xf / 2.0 ** E[:, None]
    # nearest magnitude; at an exact tie the even index (even mantissa bit)
    # wins through a bias far below any non-tie gap
    d = np.abs(np.abs(y)[..., None] - mags) + np.array([0, 1] * 4) * 1e-15
    return E, np.copysign(mags[np.argmin(d, -1)], y) * 2.0 ** E[:, None]


def test_cache_layout_and_blocks_brute_force():
    """Keys in blocks of 32 channels per token, values in blocks of 32 tokens
    per channel: the dequantized cache equals the numpy brute force, and the
    error stays within 2^(E+1) (half of E2M1's widest step, or saturation)."""
    rng = np.random.default_rng(23)
    H, T, D = 2, 96, 128
    k = rng.standard_normal((H, T, D)).astype(np.float32)
    k[:, :, 5] *= 30.0
    k[:, 7, :] = 0.0                          # a token of zeros
    v = (rng.standard_normal((H, T, D)) * rng.uniform(0.01, 50, (1, 1, D))).astype(np.float32)
    kb, vb = k.astype(np.float16), v.astype(np.float16)
    c = oracle.mx_empty_cache(D, T + 32, H)
    oracle.mx_quantize_pack(c, kb.view(np.uint16), vb.view(np.uint16), 0, T)
    kh, vh = oracle.mx_dequantize(c, 0, T)
    Ek, kref = _mx_numpy(kb.reshape(-1, 32))
    assert np.array_equal(kh.reshape(-1, 32), kref.astype(np.float32))
    assert np.array_equal(c.k_scale[:, :T].reshape(-1), Ek + 127)
    vt = vb.transpose(0, 2, 1).reshape(H, D, T // 32, 32)          # [h][d][block][32]
    Ev, vref = _mx_numpy(vt.reshape(-1, 32))
    vref = vref.reshape(H, D, T // 32, 32).reshape(H, D, T).transpose(0, 2, 1)
    assert np.array_equal(vh, vref.astype(np.float32))
    assert np.array_equal(c.v_scale[:, : T // 32].transpose(0, 2, 1).reshape(-1), Ev + 127)
    # nibble j of key word (t, w) is channel 8w + j
    for (h, t, d) in [(0, 3, 0), (1, 50, 37), (0, 95, 127)]:
        code = (int(c.k_words[h, t, d // 8]) >> (4 * (d % 8))) & 15
        assert oracle.mx_dequant(code, int(c.k_scale[h, t, d // 32])) == kh[h, t, d]
        code = (int(c.v_words[h, t // 8, d]) >> (4 * (t % 8))) & 15
        assert oracle.mx_dequant(code, int(c.v_scale[h, t // 32, d])) == vh[h, t, d]
    err_k = np.abs(kh.reshape(-1, 32) - kb.reshape(-1, 32).astype(np.float64))
    assert np.all(err_k <= 2.0 ** (Ek[:, None] + 1))


def test_attention_over_mx_cache_is_attention_over_its_dequantized_values():
    rng = np.random.default_rng(24)
    H_kv, H_q, T, D, R = 2, 8, 64, 128, 16
    k = rng.standard_normal((H_kv, T, D)).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((H_kv, T, D)).astype(np.float16).view(np.uint16)
    kr = rng.standard_normal((H_kv, R, D)).astype(np.float16)
    vr = rng.standard_normal((H_kv, R, D)).astype(np.float16)
    q = rng.standard_normal((1, H_q, D)).astype(np.float16)
    c = oracle.mx_empty_cache(D, T, H_kv)
    oracle.mx_quantize_pack(c, k, v, 0, T)
    out = oracle.mx_decode_attention(c, 1, H_q, H_kv, q.view(np.uint16), T,
                                     k_res=kr.view(np.uint16), v_res=vr.view(np.uint16), n_res=R)
    kh, vh = oracle.mx_dequantize(c, 0, T)
    g = H_q // H_kv
    for h in range(H_q):
        K = np.concatenate([kh[h // g], kr[h // g].astype(np.float32)]).astype(np.float64)
        V = np.concatenate([vh[h // g], vr[h // g].astype(np.float32)]).astype(np.float64)
        s = K @ q[0, h].astype(np.float64) / math.sqrt(D)
        p = np.exp(s - s.max())
        assert np.allclose(out[0, h], p @ V / p.sum(), rtol=0, atol=1e-12)


def test_bad_configurations_rejected():
    c = oracle.mx_empty_cache(128, 64, 1)
    x = np.zeros((1, 64, 128), np.uint16)
    for t0, n in ((16, 32), (0, 48), (32, 64)):
        with pytest.raises(ValueError):
            oracle.mx_quantize_pack(c, x, x, t0, n)
