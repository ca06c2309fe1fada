"""Byte accounting used by bench.py, pinned to the pages' numbers."""

import os

import bench
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows():
    rows = []
    for ln in open(os.path.join(GOLDEN, "kv_bytes.txt")):
        if ln.strip() and not ln.startswith("#"):
            rows.append(ln.split())
    return rows


def test_fp16_cache_size_formula():
    # KVQuant page, memory-wall section: 2*n*h*d*e bytes per token; the decode
    # byte count of an all-fp16 window reduces to the same formula
    for r in _rows()[:2]:
        layers, heads, dim, e, tokens, total = map(int, r)
        w = synth.shrink(synth.WORKLOADS["llama3_8b_t32k_2bit"], B=1, H_q=heads, H_kv=heads,
                         D=dim, T=0, R=tokens, S=0)
        per_layer = bench.decode_bytes(w) - w.B * w.H_q * w.D * 6   # drop q and out
        assert per_layer * layers == total


def test_kivi_average_bits():
    # KVQuant page, results: KIVI-2bit, group 32, 128 fp16 residual -> 3.05 bits
    bits, G, R, L, want = _rows()[2]
    got = bench.avg_bits_per_element(int(bits), int(G), int(L) - int(R), int(R))
    assert round(got, 2) == float(want)


def test_decode_bytes_of_workloads():
    W = synth.WORKLOADS
    assert bench.decode_bytes(W["llama3_8b_t32k_2bit"]) == 155_385_856
    assert bench.decode_bytes(W["tiny_t512_g32_2bit"]) == 66_304
    assert bench.decode_bytes(W["long_t1m_2bit_splitk"]) == 604_528_640
    assert bench.decode_bytes(W["llama3_8b_t8k_b32_4bit"]) == 302_776_320
    assert bench.decode_bytes(W["kitty_t128k_h64_boost16"]) == 1_303_117_824
