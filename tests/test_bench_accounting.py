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


def test_counter_csv_parse_and_copy_scale(tmp_path):
    # the counter files rocprofv3 writes name kernels with their namespaces,
    # template arguments and parameter lists; the copy kernel's reading gives
    # the scale (a 1 GiB pass read 2x too low by FETCH_SIZE on this chip)
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    rows = [
        (1, "void kvq::(anonymous namespace)::decode_f8f4_kernel<4, false, false>(kvq::DecodeArgs)", 100.0),
        (2, "void kvq::(anonymous namespace)::decode_f8f4_kernel<4, false, false>(kvq::DecodeArgs)", 110.0),
        (3, "kvq::(anonymous namespace)::merge_kernel(kvq::DecodeArgs)", 4.0),
        (4, "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda"
            "(at::TensorIteratorBase&)::{lambda(int)#1}, std::array<char*, 2ul> >(int, x)",
         bench.CALIB_COPY_BYTES / 1024 / 2),
        (5, "void at::native::unrelated_kernel<float>(float*)", 7.0),
    ]
    f = tmp_path / "fetch.csv"
    f.write_text(hdr + "".join(f'{i},"{n}",FETCH_SIZE,{v}\n' for i, n, v in rows))
    means, counts = bench._counter_means(str(f), "FETCH_SIZE")
    assert counts["decode_f8f4_kernel<4, false, false>"] == 2
    assert means["decode_f8f4_kernel<4, false, false>"] == 105.0
    assert means["merge_kernel"] == 4.0
    assert bench.COPY_KERNEL in means and "unrelated_kernel<float>" not in means
    assert bench.CALIB_COPY_BYTES / (means[bench.COPY_KERNEL] * 1024) == 2.0


def test_launches_per_step_of_workloads():
    # the library's dispatch: one launch where the split-K kernel quantizes
    # the appended group and merges in place (at most 8 parts, or 32 blocks
    # of 8 chunks in the one-chunk-per-wave geometry); Kitty's append runs at
    # the end of the blocks of a step that merges in place
    W = synth.WORKLOADS
    assert bench.launches_per_step(W["llama3_8b_t32k_2bit"], 4, True) == 1
    assert bench.launches_per_step(W["llama3_8b_t8k_b32_4bit"], 2, True) == 1
    assert bench.per_wave_chunks(W["long_t1m_2bit_splitk"], 256)
    assert bench.launches_per_step(W["long_t1m_2bit_splitk"], 256, True) == 1
    assert bench.launches_per_step(W["long_t1m_2bit_splitk"], 512, True) == 2
    assert bench.launches_per_step(W["kitty_t128k_h64_boost16"], 2, True) == 1
    assert bench.launches_per_step(W["kitty_t128k_h64_boost16"], 16, True) == 2
    assert bench.launches_per_step(W["kitty_t128k_h64_boost16"], 2, False) == 1
