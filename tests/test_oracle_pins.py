"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden/ with their citations), closed forms,
an independent implementation (numpy's binary16), exact rational arithmetic,
high-precision brute force (mpmath), or invariants.  CPU only.
"""

import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def h2f(bits):
    return float(np.array(bits, np.uint16).view(np.float16))


def f2h(x):
    return int(np.array(x, np.float16).view(np.uint16))


# --------------------------------------------------------------------------
# binary16 conversions: exhaustive against numpy's independent implementation
# --------------------------------------------------------------------------

def test_f16_to_f32_exhaustive():
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = all_bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in all_bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # signed zero survives
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


def test_f32_to_f16_rne_against_numpy():
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal(20000).astype(np.float32) * np.float32(s)
          for s in (1e-7, 1e-5, 1e-2, 1.0, 100.0, 3e4)]
    xs = np.concatenate(xs)
    # exact ties between neighbouring fp16 values in several binades, subnormal
    # ties, the overflow threshold, signed zeros
    h = np.arange(0, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, -65520.0,
                        2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -24, 3 * 2.0 ** -25,
                        5.960464477539063e-08, 6.097555160522461e-05], np.float32)
    xs = np.concatenate([xs, ties, -ties, special])
    got = np.array([oracle.f32_to_f16(float(x)) for x in xs], np.uint16)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# packing: worked examples of the KIVI and Kitty pages, closed forms, round trip
# --------------------------------------------------------------------------

def test_kivi_worked_unpack_example():
    # KIVI page, Step 4: logical column 19 at 2 bits -> word 1, shift 6, mask 0b11
    (bits, idx, word, shift, mask), = [[int(v) for v in r] for r in _rows("kivi_unpack_example.txt")]
    codes = np.zeros(32, np.uint8)
    codes[idx] = 3
    words = oracle.pack(codes, bits)
    assert words[word] == mask << shift
    assert np.count_nonzero(words) == 1
    for c in range(4):
        codes[idx] = c
        assert oracle.unpack(oracle.pack(codes, bits), 32, bits)[idx] == c


def test_kitty_byte_shifts():
    # Kitty page, Algorithm 1: byte k of the 2-bit stream holds four consecutive
    # codes at shifts 0, 2, 4, 6 -- the same bytes as least-significant-first int32
    # packing on a little-endian machine
    shifts = [int(r[1]) for r in _rows("kitty_byte_shifts.txt")]
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, 64, dtype=np.uint8)
    b = oracle.pack(codes, 2).view(np.uint8)
    for k in range(16):
        for p in range(4):
            assert (b[k] >> shifts[p]) & 3 == codes[4 * k + p]


def test_pack_closed_forms():
    assert oracle.pack(np.tile(np.arange(4, dtype=np.uint8), 4), 2)[0] == 0xE4E4E4E4
    assert oracle.pack(np.arange(8, dtype=np.uint8), 4)[0] == 0x76543210
    assert oracle.pack(np.array([0x12, 0x34, 0x56, 0x78], np.uint8), 8)[0] == 0x78563412
    assert oracle.pack(np.full(16, 3, np.uint8), 2)[0] == 0xFFFFFFFF


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    n = 32 * 37
    codes = rng.integers(0, 1 << bits, n, dtype=np.uint8)
    assert np.array_equal(oracle.unpack(oracle.pack(codes, bits), n, bits), codes)


# --------------------------------------------------------------------------
# one group: hand-worked examples, exact-rational rounding, guard, bound
# --------------------------------------------------------------------------

def test_quant_hand_examples():
    for r in open(os.path.join(GOLDEN, "quant_examples.txt")):
        if not r.strip() or r.startswith("#"):
            continue
        head, xs, ms, codes, deq = [p.split() for p in r.split("|")]
        bits = int(head[1])
        x = np.array([int(v, 16) for v in xs], np.uint16)
        mn, s, q = oracle.quantize_group(x, bits)
        assert (mn, s) == (int(ms[0], 16), int(ms[1], 16)), head[0]
        assert list(q) == [int(c) for c in codes], head[0]
        assert [oracle.dequant(int(c), s, mn) for c in q] == [float(v) for v in deq], head[0]


def _exact_nearest_even(y: Fraction) -> int:
    f = math.floor(y)
    d = y - f
    if d > Fraction(1, 2):
        return f + 1
    if d < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_are_nearest_grid_points(bits):
    """Codes equal exact rational round(clamp((x - mn)/s)), ties to even, except
    inside a tiny neighbourhood of a tie where fp32 rounding may decide."""
    maxq = (1 << bits) - 1
    rng = np.random.default_rng(100 + bits)
    near_tie = 0
    for trial in range(300):
        n = int(rng.integers(2, 40))
        scale = 10.0 ** rng.uniform(-3, 2)
        x = (rng.standard_normal(n) * scale).astype(np.float16).view(np.uint16)
        mn, s, q = oracle.quantize_group(x, bits)
        xs = [Fraction(h2f(v)) for v in x]
        assert Fraction(h2f(mn)) == min(xs)
        # stored scale: fp16 nearest to (max-min)/maxq up to one fp32 rounding
        exact_s = (max(xs) - min(xs)) / maxq
        if exact_s == 0:
            assert s == 0 and not q.any()
            continue
        sf = Fraction(h2f(s))
        # fp16 spacing at exact_s: 2^(e-11) for a normal value, 2^-24 below 2^-14
        # (8-bit scales, range/255, often fall into the subnormal range)
        ulp = max(Fraction(2) ** (math.frexp(float(exact_s))[1] - 11), Fraction(1, 1 << 24))
        assert abs(sf - exact_s) <= ulp / 2 * (1 + Fraction(1, 1 << 12))
        for xv, qv in zip(xs, q):
            y = min(max((xv - min(xs)) / sf, Fraction(0)), Fraction(maxq))
            want = _exact_nearest_even(y)
            if abs(y - math.floor(y) - Fraction(1, 2)) < Fraction(1, 1 << 18):
                near_tie += 1
                assert qv in (math.floor(y), math.floor(y) + 1)
            else:
                assert qv == want
    assert near_tie < 50


def test_guard_constant_and_signed_zero_groups():
    for x in ([0x3E00] * 5, [0x8000, 0x0000, 0x8000], [0x0000] * 3):
        mn, s, q = oracle.quantize_group(np.array(x, np.uint16), 2)
        assert s == 0 and not q.any()
        assert oracle.dequant(0, s, mn) == h2f(mn)
    # -0 sorts below +0, independent of order
    assert oracle.group_minmax(np.array([0x0000, 0x8000], np.uint16)) == (0x8000, 0x0000)
    assert oracle.group_minmax(np.array([0x8000, 0x0000], np.uint16)) == (0x8000, 0x0000)
    # a range so small that range/maxq underflows fp16 to zero takes the guard
    mn, s, q = oracle.quantize_group(np.array([0x0000, 0x0001], np.uint16), 2)
    assert s == 0 and not q.any()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exactly_representable_groups_roundtrip(bits):
    """Values mn + k*2^e covering codes 0 and maxq: scale 2^e, dequant exact."""
    maxq = (1 << bits) - 1
    rng = np.random.default_rng(7 + bits)
    ran = 0
    for e in (-6, -2, 0, 3):
        for mn in (-3.0, 0.0, 1.25):
            k = rng.integers(0, maxq + 1, 20)
            k[0], k[1] = 0, maxq
            vals = [mn + int(kk) * 2.0 ** e for kk in k]
            x = np.array([f2h(v) for v in vals], np.uint16)
            if [h2f(v) for v in x] != vals:
                continue   # not every value fits fp16's 11 significant bits (8-bit codes)
            ran += 1
            m, s, q = oracle.quantize_group(x, bits)
            assert h2f(s) == 2.0 ** e and h2f(m) == mn
            assert list(q) == list(k)
            assert [oracle.dequant(int(c), s, m) for c in q] == [h2f(v) for v in x]
    assert ran >= 6


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequant_error_bound(bits):
    """|x - dequant| <= s/2 (plus the fp32/fp16 rounding slop) for normal s."""
    rng = np.random.default_rng(11 + bits)
    for trial in range(200):
        n = 128
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-2, 2)).astype(np.float16)
        mn, s, q = oracle.quantize_group(x.view(np.uint16), bits)
        sf = h2f(s)
        assert sf >= 2.0 ** -14
        err = np.abs(x.astype(np.float64) - np.array([oracle.dequant(int(c), s, mn) for c in q]))
        assert np.all(err <= sf / 2 * (1 + 2.0 ** -20) + 2.0 ** -23 * np.abs(x.astype(np.float64)))


# --------------------------------------------------------------------------
# whole-cache helpers
# --------------------------------------------------------------------------

def _rand_src(rng, heads, n, D, outliers=()):
    k = rng.standard_normal((heads, n, D)).astype(np.float32)
    for c, m in outliers:
        k[:, :, c] *= m
    v = rng.standard_normal((heads, n, D)).astype(np.float32)
    return k.astype(np.float16).view(np.uint16), v.astype(np.float16).view(np.uint16)


def test_cache_layout_matches_group_primitive():
    """Cache entries equal the single-group primitive applied to the slices the
    layout names: K per channel over G tokens, packed along channels; V per
    token over G channels, packed along tokens."""
    rng = np.random.default_rng(3)
    for bits, G in ((2, 32), (4, 64), (2, 128)):
        D, heads, T = 128, 2, 256
        c = oracle.empty_cache(bits, G, D, 0, T, heads)
        k, v = _rand_src(rng, heads, T, D, [(5, 12.0)])
        oracle.quantize_pack(c, k, v, 0, T // G)
        fpi = 32 // bits
        for hd in range(heads):
            for g in (0, T // G - 1):
                for d in (0, 5, 77, 127):
                    mn, s, q = oracle.quantize_group(k[hd, g * G:(g + 1) * G, d], bits)
                    assert (c.k_min[hd, g, d], c.k_scale[hd, g, d]) == (mn, s)
                    for j in (0, G - 1):
                        t = g * G + j
                        w = c.k_words[hd, t, d // fpi]
                        assert (w >> (bits * (d % fpi))) & ((1 << bits) - 1) == q[j]
            for t in (0, 31, T - 1):
                for cg in range(D // G):
                    mn, s, q = oracle.quantize_group(v[hd, t, cg * G:(cg + 1) * G], bits)
                    assert (c.v_min[hd, t, cg], c.v_scale[hd, t, cg]) == (mn, s)
                    for d in (cg * G, cg * G + G - 1):
                        w = c.v_words[hd, t // fpi, d]
                        assert (w >> (bits * (t % fpi))) & ((1 << bits) - 1) == q[d - cg * G]


def test_append_matches_bulk():
    """Quantizing group by group (streaming append) equals one bulk call."""
    rng = np.random.default_rng(4)
    bits, G, D, heads, T = 2, 64, 128, 3, 256
    k, v = _rand_src(rng, heads, T, D)
    bulk = oracle.empty_cache(bits, G, D, 0, T, heads)
    oracle.quantize_pack(bulk, k, v, 0, T // G)
    step = oracle.empty_cache(bits, G, D, 0, T, heads)
    for g in range(T // G):
        oracle.quantize_pack(step, k[:, g * G:(g + 1) * G], v[:, g * G:(g + 1) * G], g, 1)
    for name in ("k_words", "k_scale", "k_min", "v_words", "v_scale", "v_min"):
        assert np.array_equal(getattr(bulk, name), getattr(step, name)), name


# --------------------------------------------------------------------------
# Kitty channel-wise boost
# --------------------------------------------------------------------------

def _np_quant(xh, maxq):
    """One min-max group restated in numpy, independently of the oracle (KIVI
    page, Step 1, with the fp32 reading): min and max under the order
    -0 < +0, range and quotient in IEEE fp32, the scale rounded to fp16, codes
    round-half-even(clamp((x - min)/scale, 0, maxq)); a zero scale gives code 0.
    Returns (min bits, scale bits, codes)."""
    xh = np.asarray(xh, np.float16)
    b = xh.view(np.uint16).astype(np.int64)
    key = np.where(b & 0x8000, 0x7FFF - (b & 0x7FFF), 0x8000 + b)
    mn, mx = xh[np.argmin(key)], xh[np.argmax(key)]
    s = np.float16((np.float32(mx) - np.float32(mn)) / np.float32(maxq))
    if s == 0:
        codes = np.zeros(len(xh), np.uint8)
    else:
        y = (xh.astype(np.float32) - np.float32(mn)) / np.float32(s)
        codes = np.rint(np.clip(y, np.float32(0), np.float32(maxq))).astype(np.uint8)
    return int(np.array(mn).view(np.uint16)), int(np.array(s).view(np.uint16)), codes


def _field(words, idx, bits):
    """Code idx of a least-significant-first packed row (numpy shift-and-mask)."""
    per = 32 // bits
    return (words[..., idx // per] >> np.uint32(bits * (idx % per))) & np.uint32((1 << bits) - 1)


@pytest.mark.parametrize("nb,G", [(0, 64), (0, 128), (16, 64), (16, 128), (32, 64), (32, 128)])
def test_kitty_partial_boost_codes_high_bits_and_dequant(nb, G):
    """Kitty page, 4.1 (a key page is a dense tensor of every channel's low two
    bits, a compact (D_boost, G) tensor of the boosted channels' high two bits
    and a per-channel index with a sentinel) and 4.2, Algorithm 1 (X = lo |
    hi << 2, X * scale + zero), checked channel by channel against the numpy
    restatement of the quantizer with 0 < n_boost < D, where a boosted row is
    not its channel:
      * the boosted set is the n_boost channels of largest fp32 range, ties to
        the lower channel, and row r is the r-th of them in ascending order;
      * each channel's scale and min are those of its own width (15 levels
        boosted, 3 otherwise), and its dense 2-bit field holds code & 3;
      * the high-bits word (t, r // 16) holds code >> 2 of row r's channel at
        bit 2 (r % 16), for every token t of the group;
      * the dequantized key is (lo | hi << 2) * scale + min in fp32.
    n_boost = 0 is plain 2-bit KIVI: every channel against the same numpy
    quantizer at 3 levels."""
    rng = np.random.default_rng(40 + nb + G)
    D, T, heads = 128, 256, 2
    k, v = _rand_src(rng, heads, T, D, [(2, 20.0), (9, 15.0), (33, 18.0), (70, 12.0),
                                        (101, 25.0), (126, 14.0)])
    c = oracle.empty_cache(2, G, D, nb, T, heads)
    oracle.quantize_pack(c, k, v, 0, T // G)
    kk, vv = oracle.dequantize(c, 0, T // G)
    kf = k.view(np.float16)
    vf = v.view(np.float16)
    for hd in range(heads):
        for g in range(T // G):
            blk = kf[hd, g * G:(g + 1) * G]
            rng32 = blk.max(0).astype(np.float32) - blk.min(0).astype(np.float32)
            boosted = sorted(sorted(range(D), key=lambda d: (-float(rng32[d]), d))[:nb])
            rank = {d: r for r, d in enumerate(boosted)}
            assert boosted != list(range(nb)) or nb == 0   # rows differ from channels
            toks = slice(g * G, (g + 1) * G)
            for d in range(D):
                maxq = 15 if d in rank else 3
                mn, s, q = _np_quant(blk[:, d], maxq)
                assert (int(c.k_min[hd, g, d]), int(c.k_scale[hd, g, d])) == (mn, s), (hd, g, d)
                lo = _field(c.k_words[hd, toks], d, 2)
                assert np.array_equal(lo, q & 3), (hd, g, d)
                code = lo.astype(np.uint32)
                if nb:
                    assert int(c.k_bidx[hd, g, d]) == rank.get(d, nb)
                if d in rank:
                    r = rank[d]
                    hi = _field(c.k_hi[hd, toks], r, 2)
                    assert np.array_equal(hi, q >> 2), (hd, g, d, r)
                    code = code | (hi << np.uint32(2))
                want = (code.astype(np.float32) * np.float16(np.uint16(s).view(np.float16)).astype(np.float32)
                        + np.float32(np.uint16(mn).view(np.float16)))
                assert np.array_equal(kk[hd, toks, d].view(np.uint32), want.view(np.uint32)), (hd, g, d)
    # values stay plain 2-bit per token (Kitty page, 3.3: V2)
    for hd in range(heads):
        for t in (0, 77, T - 1):
            for cg in range(D // G):
                mn, s, q = _np_quant(vf[hd, t, cg * G:(cg + 1) * G], 3)
                assert (int(c.v_min[hd, t, cg]), int(c.v_scale[hd, t, cg])) == (mn, s)
                got = [int(_field(c.v_words[hd, :, d], t, 2)) for d in range(cg * G, (cg + 1) * G)]
                assert got == list(q)


def test_key_words_bridge_to_kivi_token_axis_packing():
    """KIVI page, Step 2 packs key codes along tokens, [T/16, D] at 2 bits: word
    (w, d) holds token 16 w + j of channel d at bit 2 j; Step 4's worked example
    finds logical column 19 in word 1 at shift 6 (tests/golden/
    kivi_unpack_example.txt).  The cache packs the same codes along channels.
    Re-packing the cache's codes of each channel along tokens with the page's
    shift-or (numpy) must give the page's words built from the numpy quantizer's
    codes, and token 19 of every channel must sit in word 1 at shift 6: the
    bit-exact words of the cache are a fixed transposition of the page's words,
    with the same codes."""
    (bits, idx, word, shift, mask), = [[int(x) for x in r] for r in _rows("kivi_unpack_example.txt")]
    rng = np.random.default_rng(41)
    D, G, T = 128, 32, 64
    k, v = _rand_src(rng, 1, T, D, [(3, 15.0), (17, 15.0)])
    c = oracle.empty_cache(bits, G, D, 0, T, 1)
    oracle.quantize_pack(c, k, v, 0, T // G)
    kf = k.view(np.float16)[0]
    page_codes = np.zeros((T, D), np.uint32)           # quant_kcache's code[t][d]
    for g in range(T // G):
        for d in range(D):
            page_codes[g * G:(g + 1) * G, d] = _np_quant(kf[g * G:(g + 1) * G, d], 3)[2]
    per = 32 // bits

    def pack_tokens(codes):                              # pack_tensor along tokens
        w = np.zeros((T // per, D), np.uint32)
        for j in range(per):
            w |= codes[j::per] << np.uint32(bits * j)
        return w

    page_words = pack_tokens(page_codes)
    cache_codes = np.stack([_field(c.k_words[0], d, bits) for d in range(D)], -1)   # [T][D]
    assert np.array_equal(pack_tokens(cache_codes.astype(np.uint32)), page_words)
    assert np.array_equal((page_words[word] >> np.uint32(shift)) & np.uint32(mask), page_codes[idx])
    # the same code read straight from the cache's channel-axis word
    for d in (0, 3, 17, 127):
        assert (int(c.k_words[0, idx, d // per]) >> (bits * (d % per))) & mask == \
            (int(page_words[word, d]) >> shift) & mask


def test_value_words_bridge_to_channel_axis_packing():
    """Values are quantized per token over G channels (KIVI page, Step 1) and
    the cache packs them along tokens; re-packing its codes of each token along
    channels (least significant first, as pack_tensor) gives the words built
    from the numpy quantizer's per-token codes."""
    rng = np.random.default_rng(42)
    D, G, T = 128, 64, 64
    for bits in (2, 4):
        k, v = _rand_src(rng, 1, T, D)
        c = oracle.empty_cache(bits, G, D, 0, T, 1)
        oracle.quantize_pack(c, k, v, 0, T // G)
        vf = v.view(np.float16)[0]
        maxq = (1 << bits) - 1
        page = np.concatenate([np.stack([_np_quant(vf[t, cg * G:(cg + 1) * G], maxq)[2]
                                         for t in range(T)]) for cg in range(D // G)], 1)
        cache_codes = np.stack([[int(_field(c.v_words[0, :, d], t, bits)) for d in range(D)]
                                for t in range(T)])
        assert np.array_equal(cache_codes, page.astype(np.int64))
        per = 32 // bits
        chan_words = np.zeros((T, D // per), np.uint32)
        for j in range(per):
            chan_words |= page[:, j::per].astype(np.uint32) << np.uint32(bits * j)
        for t in range(T):
            assert list(oracle.unpack(chan_words[t], D, bits)) == [int(x) for x in cache_codes[t]]


def test_kitty_all_channels_boosted_equals_4bit():
    """n_boost = D: every key channel is 4-bit; lo | hi << 2 (Kitty Algorithm 1)
    reproduces the plain 4-bit codes and the dequantized keys bit for bit."""
    rng = np.random.default_rng(6)
    D, G, T, heads = 128, 64, 128, 2
    k, v = _rand_src(rng, heads, T, D, [(3, 15.0)])
    kit = oracle.empty_cache(2, G, D, D, T, heads)
    oracle.quantize_pack(kit, k, v, 0, T // G)
    p4 = oracle.empty_cache(4, G, D, 0, T, heads)
    oracle.quantize_pack(p4, k, v, 0, T // G)
    assert np.array_equal(kit.k_scale, p4.k_scale) and np.array_equal(kit.k_min, p4.k_min)
    assert np.array_equal(kit.k_bidx, np.broadcast_to(np.arange(D, dtype=np.uint8), kit.k_bidx.shape))
    lo = np.stack([(kit.k_words[..., d // 16] >> (2 * (d % 16))) & 3 for d in range(D)], -1)
    hi = np.stack([(kit.k_hi[..., d // 16] >> (2 * (d % 16))) & 3 for d in range(D)], -1)
    q4 = np.stack([(p4.k_words[..., d // 8] >> (4 * (d % 8))) & 15 for d in range(D)], -1)
    assert np.array_equal(lo | (hi << 2), q4)
    kk, _ = oracle.dequantize(kit, 0, T // G)
    k4, _ = oracle.dequantize(p4, 0, T // G)
    assert np.array_equal(kk, k4)


def test_kitty_boosted_set_is_top_range():
    """Boosted channels are the n_boost of largest per-group range (computed
    here independently in float64 from the fp16 source), rows ascending."""
    rng = np.random.default_rng(8)
    D, G, T, heads, nb = 128, 128, 256, 2, 16
    k, v = _rand_src(rng, heads, T, D, [(c, 20.0) for c in (1, 40, 41, 99, 100, 120, 121, 127)])
    c = oracle.empty_cache(2, G, D, nb, T, heads)
    oracle.quantize_pack(c, k, v, 0, T // G)
    kf = k.view(np.float16).astype(np.float64)
    for hd in range(heads):
        for g in range(T // G):
            blk = kf[hd, g * G:(g + 1) * G]
            rng_d = blk.max(0) - blk.min(0)
            top = np.sort(np.argsort(-rng_d, kind="stable")[:nb])
            bidx = c.k_bidx[hd, g]
            assert list(np.nonzero(bidx < nb)[0]) == list(top)
            assert list(bidx[top]) == list(range(nb))
            assert np.all(bidx[bidx >= nb] == nb)
            # boosted channels use 15 levels, the others 3
            for d in range(D):
                maxq = 15 if bidx[d] < nb else 3
                m, s, _ = oracle.quantize_group(k[hd, g * G:(g + 1) * G, d], 4 if maxq == 15 else 2)
                assert (c.k_min[hd, g, d], c.k_scale[hd, g, d]) == (m, s)


def _boosted(c, hd, g, nb):
    return list(np.nonzero(c.k_bidx[hd, g] < nb)[0])


def test_kitty_magnitude_score_hand_group():
    """Kitty page, section 3.2: with the magnitude score the boosted channels
    are those of largest mean |x| over the group, not of largest range.
    Channels 0..15 are one spike of 1000 among zeros (range 1000, mean |x|
    1000/128); channels 16..23 are constant 50, channels 24..31 constant -60
    (range 0, mean |x| 50 and 60); the rest lie in (-1, 1)."""
    rng = np.random.default_rng(12)
    D, G, nb = 128, 128, 16
    k = (rng.random((1, G, D)) * 1.8 - 0.9).astype(np.float32)
    k[0, :, :16] = 0.0
    k[0, 5, :16] = 1000.0
    k[0, :, 16:24] = 50.0
    k[0, :, 24:32] = -60.0
    kb = k.astype(np.float16).view(np.uint16)
    vb = np.zeros_like(kb)
    by_range = oracle.empty_cache(2, G, D, nb, G, 1)
    oracle.quantize_pack(by_range, kb, vb, 0, 1)
    assert _boosted(by_range, 0, 0, nb) == list(range(16))
    by_mag = oracle.empty_cache(2, G, D, nb, G, 1, score=1)
    oracle.quantize_pack(by_mag, kb, vb, 0, 1)
    assert _boosted(by_mag, 0, 0, nb) == list(range(16, 32))
    assert list(by_mag.k_bidx[0, 0, 16:32]) == list(range(16))
    # a constant channel has scale 0 and decodes to its value exactly
    kk, _ = oracle.dequantize(by_mag, 0, 1)
    assert np.all(kk[0, :, 16:24] == 50.0) and np.all(kk[0, :, 24:32] == -60.0)


def test_kitty_magnitude_score_ties_and_sign():
    """Equal sums of |x| tie to the lower channel whatever the signs; a
    negative channel counts by its magnitude."""
    D, G, nb = 128, 64, 16
    k = np.ones((1, G, D), np.float32)
    k[0, ::2, :] = -1.0                      # every channel: mean |x| = 1
    k[0, :, 100] = -3.0                      # largest magnitude, all negative
    kb = k.astype(np.float16).view(np.uint16)
    c = oracle.empty_cache(2, G, D, nb, G, 1, score=1)
    oracle.quantize_pack(c, kb, np.zeros_like(kb), 0, 1)
    assert _boosted(c, 0, 0, nb) == list(range(15)) + [100]


def test_kitty_magnitude_score_brute_force():
    """Random groups: the boosted set equals the top n_boost channels by the
    sum of |x| (exact rationals here), ties to the lower channel; with
    n_boost = D both scores give the plain 4-bit cache."""
    rng = np.random.default_rng(13)
    D, G, T, heads = 128, 32, 128, 2
    k, v = _rand_src(rng, heads, T, D, [(7, 12.0), (64, 9.0)])
    for nb in (16, 32):
        c = oracle.empty_cache(2, G, D, nb, T, heads, score=1)
        oracle.quantize_pack(c, k, v, 0, T // G)
        for hd in range(heads):
            for g in range(T // G):
                blk = k[hd, g * G:(g + 1) * G]
                sums = [sum(Fraction(abs(float(x))) for x in blk[:, d].view(np.float16))
                        for d in range(D)]
                order = sorted(range(D), key=lambda d: (-sums[d], d))
                assert _boosted(c, hd, g, nb) == sorted(order[:nb])
    full = oracle.empty_cache(2, G, D, D, T, heads, score=1)
    oracle.quantize_pack(full, k, v, 0, T // G)
    p4 = oracle.empty_cache(4, G, D, 0, T, heads)
    oracle.quantize_pack(p4, k, v, 0, T // G)
    assert np.array_equal(oracle.dequantize(full, 0, T // G)[0], oracle.dequantize(p4, 0, T // G)[0])


@pytest.mark.parametrize("kb,vb", [(2, 4), (4, 2), (2, 8)])
def test_mixed_widths_equal_their_uniform_parts(kb, vb):
    """Kitty page, section 3.1 (K2V4, K4V2): keys of a mixed cache are the
    uniform kb-bit cache's keys and its values the uniform vb-bit cache's
    values, word for word and after dequantization; decode over it equals
    attention over those dequantized keys and values."""
    rng = np.random.default_rng(14)
    D, G, T, heads = 128, 128, 256, 2
    k, v = _rand_src(rng, heads, T, D, [(3, 15.0)])
    mix = oracle.empty_cache(kb, G, D, 0, T, heads, v_bits=vb)
    oracle.quantize_pack(mix, k, v, 0, T // G)
    ck = oracle.empty_cache(kb, G, D, 0, T, heads)
    oracle.quantize_pack(ck, k, v, 0, T // G)
    cv = oracle.empty_cache(vb, G, D, 0, T, heads)
    oracle.quantize_pack(cv, k, v, 0, T // G)
    assert mix.v_words.shape == (heads, T * vb // 32, D)
    for f in ("k_words", "k_scale", "k_min"):
        assert np.array_equal(getattr(mix, f), getattr(ck, f)), f
    for f in ("v_words", "v_scale", "v_min"):
        assert np.array_equal(getattr(mix, f), getattr(cv, f)), f
    km, vm = oracle.dequantize(mix, 0, T // G)
    assert np.array_equal(km, oracle.dequantize(ck, 0, T // G)[0])
    assert np.array_equal(vm, oracle.dequantize(cv, 0, T // G)[1])
    q = rng.standard_normal((1, 4, D)).astype(np.float16).view(np.uint16)
    out = oracle.decode_attention(mix, 1, 4, 2, q, T)
    sm = 1.0 / math.sqrt(D)
    for h in range(4):
        ref = oracle.attention_fp64(q[0, h].view(np.float16).astype(np.float64),
                                    km[h // 2].astype(np.float64), vm[h // 2].astype(np.float64), sm)
        assert np.allclose(out[0, h], ref, rtol=0, atol=1e-12)


def test_mixed_widths_reject_bad_configurations():
    """A value width that does not divide the group into whole words, or a
    Kitty boost with values wider than 2 bits, is refused."""
    rng = np.random.default_rng(15)
    k, v = _rand_src(rng, 1, 64, 128)
    with pytest.raises(ValueError):
        c = oracle.empty_cache(2, 64, 128, 16, 64, 1, v_bits=4)
        c.k_hi = np.zeros((1, 64, 1), np.uint32)
        oracle.quantize_pack(c, k, v, 0, 1)
    with pytest.raises(ValueError):
        oracle.quantize_pack(oracle.empty_cache(2, 64, 128, 0, 64, 1, v_bits=3), k, v, 0, 1)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _brute_attention(q, K, V, sm):
    """50-digit brute force, no max subtraction."""
    mpmath.mp.dps = 50
    w = [mpmath.exp(mpmath.mpf(sm) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                                for a, b in zip(q, k))) for k in K]
    Z = mpmath.fsum(w)
    return np.array([float(mpmath.fsum(wi * mpmath.mpf(float(vi[d])) for wi, vi in zip(w, V)) / Z)
                     for d in range(len(q))])


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(9)
    for n in (1, 2, 5, 8):
        q = rng.standard_normal(4)
        K = rng.standard_normal((n, 4)) * 3
        V = rng.standard_normal((n, 4))
        got = oracle.attention_fp64(q, K, V, 0.5)
        assert np.allclose(got, _brute_attention(q, K, V, 0.5), rtol=1e-12, atol=1e-13)


def test_attention_uniform_logits_is_mean():
    rng = np.random.default_rng(10)
    K = np.tile(rng.standard_normal(8), (37, 1))
    V = rng.standard_normal((37, 8))
    got = oracle.attention_fp64(rng.standard_normal(8), K, V, 0.3)
    assert np.allclose(got, V.mean(0), rtol=1e-13, atol=1e-14)


def test_attention_split_merge_identity():
    rng = np.random.default_rng(11)
    q = rng.standard_normal(16)
    K = rng.standard_normal((1000, 16)) * 2
    V = rng.standard_normal((1000, 16))
    ref = oracle.attention_fp64(q, K, V, 0.25)
    for chunk in (1, 7, 128, 999, 1000, 4096):
        assert np.allclose(oracle.attention_split_merge(q, K, V, 0.25, chunk), ref,
                           rtol=0, atol=1e-12)


def _windows(rng, heads, n, D):
    k = (rng.standard_normal((heads, n, D)) * 2).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((heads, n, D)).astype(np.float16).view(np.uint16)
    return k, v


def test_decode_all_residual_is_fp16_attention():
    """No quantized tokens: decode = plain attention over the fp16 window
    (brute force), default scale 1/sqrt(D)."""
    rng = np.random.default_rng(12)
    D, n = 16, 6
    c = oracle.empty_cache(2, 16, D, 0, 16, 1)
    kr, vr = _windows(rng, 1, n, D)
    q = rng.standard_normal((1, 1, D)).astype(np.float16).view(np.uint16)
    out = oracle.decode_attention(c, 1, 1, 1, q, 0, k_res=kr, v_res=vr, n_res=n)
    qf = q.view(np.float16).astype(np.float64)[0, 0]
    ref = _brute_attention(qf, kr[0].view(np.float16), vr[0].view(np.float16), 1 / math.sqrt(D))
    assert np.allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)


def test_decode_exact_cache_equals_fp16_window():
    """Exactly representable groups dequantize to the source values, so decode
    over the quantized cache equals decode over the same tokens held fp16 --
    bit for bit.  Also pins the GQA head mapping (kv = h // (H_q/H_kv)),
    the sink window and token-order invariance."""
    rng = np.random.default_rng(13)
    bits, G, D, T = 2, 32, 64, 96
    B, H_kv, H_q = 2, 2, 6
    heads = B * H_kv
    # K: per channel values mn_d + k*2^e_d; V: per token mn_t + k*2^e_t, with
    # codes 0 and 3 present in every group
    kq = rng.integers(0, 4, (heads, T, D))
    kq[:, ::G, :], kq[:, 1::G, :] = 0, 3
    ke = rng.integers(-3, 2, (heads, T // G, 1, D)).astype(np.float64)
    km = rng.integers(-8, 8, (heads, T // G, 1, D)) / 4
    kval = (km + kq.reshape(heads, T // G, G, D) * 2.0 ** ke).reshape(heads, T, D)
    vq = rng.integers(0, 4, (heads, T, D))
    vq[:, :, 0::G], vq[:, :, 1::G] = 0, 3   # both ends of every channel group
    ve = rng.integers(-3, 1, (heads, T, 1)).astype(np.float64)
    vm = rng.integers(-8, 8, (heads, T, 1)) / 4
    vval = vm + vq * 2.0 ** ve
    k16 = kval.astype(np.float16).view(np.uint16)
    v16 = vval.astype(np.float16).view(np.uint16)
    assert np.array_equal(k16.view(np.float16).astype(np.float64), kval)
    c = oracle.empty_cache(bits, G, D, 0, T, heads)
    oracle.quantize_pack(c, k16, v16, 0, T // G)
    kd, vd = oracle.dequantize(c, 0, T // G)
    assert np.array_equal(kd.astype(np.float64), kval) and np.array_equal(vd.astype(np.float64), vval)
    q = rng.standard_normal((B, H_q, D)).astype(np.float16).view(np.uint16)
    ks, vs = _windows(rng, heads, 3, D)
    quant = oracle.decode_attention(c, B, H_q, H_kv, q, T, k_sink=ks, v_sink=vs, n_sink=3)
    # same tokens, all held in the fp16 residual window (sink first, then cache)
    kr = np.concatenate([ks, k16], 1)
    vr = np.concatenate([vs, v16], 1)
    empty = oracle.empty_cache(bits, G, D, 0, T, heads)
    full = oracle.decode_attention(empty, B, H_q, H_kv, q, 0, k_res=kr, v_res=vr, n_res=T + 3)
    assert np.array_equal(quant, full)
    # per-head brute force fixes the GQA mapping
    g = H_q // H_kv
    for b in range(B):
        for h in range(H_q):
            hd = b * H_kv + h // g
            ref = _brute_attention(q[b, h].view(np.float16).astype(np.float64),
                                   kr[hd].view(np.float16), vr[hd].view(np.float16),
                                   1 / math.sqrt(D)) if (b, h) in ((0, 0), (1, 5)) else None
            if ref is not None:
                assert np.allclose(quant[b, h], ref, rtol=1e-11, atol=1e-12)
    # token order does not matter (reverse the window)
    rev = oracle.decode_attention(empty, B, H_q, H_kv, q, 0, k_res=kr[:, ::-1].copy(),
                                  v_res=vr[:, ::-1].copy(), n_res=T + 3)
    assert np.allclose(rev, full, rtol=0, atol=1e-13)


def test_decode_mha_equals_per_head_attention():
    """H_q == H_kv: each query head attends its own kv head."""
    rng = np.random.default_rng(14)
    bits, G, D, T, heads = 4, 32, 32, 64, 3
    k, v = _rand_src(rng, heads, T, D)
    c = oracle.empty_cache(bits, G, D, 0, T, heads)
    oracle.quantize_pack(c, k, v, 0, T // G)
    kd, vd = oracle.dequantize(c, 0, T // G)
    q = rng.standard_normal((1, heads, D)).astype(np.float16).view(np.uint16)
    out = oracle.decode_attention(c, 1, heads, heads, q, T, sm=0.2)
    for h in range(heads):
        ref = _brute_attention(q[0, h].view(np.float16).astype(np.float64), kd[h], vd[h], 0.2)
        assert np.allclose(out[0, h], ref, rtol=1e-11, atol=1e-12)
