"""Decode-step benchmark of the low-bit KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: one decode-attention
step over the packed cache + fp16 windows (split-K, log-sum-exp merge) and
the append-group quantize+pack of the full fp16 residual group (the cache's
streaming update), as one kvq_decode_step call.  For plain 2-bit codes with
4..8 chunks per head the library runs that step as a single kernel launch.
Inputs are seeded synthetic tensors already resident in HBM.  To measure HBM rather than the 256 MB Infinity Cache, the
steps rotate over several independent copies of the packed cache (total well
above the cache size).

Prints one JSON line:  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, vendor figure
MALL_BYTES = 256 << 20       # MI355X Infinity Cache
DEFAULT_WORKLOAD = "llama3_8b_t32k_2bit"


# ----------------------------------------------------------------------------
# algorithmic bytes (what the method itself must move)
# ----------------------------------------------------------------------------

def decode_bytes(w) -> int:
    """Bytes one decode step must read/write: packed codes, fp16 scale+min per
    group, Kitty high words + index, the fp16 sink/residual windows, q (fp16)
    and the output (fp32).  Split-K partials are not counted."""
    T, D, G, b = w.T, w.D, w.G, w.bits
    per_head = (T * D * b // 8            # key codes
                + (T // G) * D * 4        # key scale + min (fp16 each)
                + T * D * b // 8          # value codes
                + T * (D // G) * 4        # value scale + min
                + (T * w.n_boost * 2 // 8 + (T // G) * D if w.n_boost else 0)  # Kitty
                + (w.S + w.R) * D * 4)    # fp16 K and V windows
    return w.heads * per_head + w.B * w.H_q * D * (2 + 4)


def append_bytes(w) -> int:
    """Bytes of the append-group quantize: read one fp16 group of K and V, write
    its codes and metadata."""
    G, D, b = w.G, w.D, w.bits
    per_head = (2 * G * D * 2 + 2 * G * D * b // 8 + D * 4 + G * (D // G) * 4
                + (G * w.n_boost * 2 // 8 + D if w.n_boost else 0))
    return w.heads * per_head


def avg_bits_per_element(bits: int, G: int, T: int, R: int) -> float:
    """Average stored bits per K/V element of a cache with T quantized tokens
    (codes + fp16 scale and min per group of G) and R fp16 residual tokens."""
    quant = bits + 32.0 / G
    return (quant * T + 16.0 * R) / (T + R)


# ----------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters (FETCH_SIZE / WRITE_SIZE, KiB per
# dispatch), scaled by what the same counters read for a plain copy of known
# size.  The figures live in a text file under profiles/ together with a hash
# of the kernel sources they were taken from; a changed source voids them.
# ----------------------------------------------------------------------------

CALIB_COPY_BYTES = 1 << 30
COPY_KERNEL = "bitwise_not"       # the calibration pass: dst = ~src over 1 GiB of int32


def split_kernel(w) -> str:
    """Name of the split-K kernel the library launches for this workload (the
    dispatch rule of the library: matrix cores for GQA 4/8 and G 128, fp8 x fp4
    for 2-bit codes, plain or with the 16-channel Kitty boost, fp16 for plain
    4-bit codes; the vector-ALU kernel otherwise)."""
    if w.G == 128 and w.gqa in (4, 8):
        if w.bits == 2 and w.n_boost in (0, 16):
            return "decode_f8f4_kernel"
        if w.bits == 4 and w.n_boost == 0:
            return "decode_mfma_kernel"
    return "decode_valu_kernel"


def compute_dtype(w) -> str:
    """The arithmetic the step's kernel computes in (not a precision claim)."""
    kern = split_kernel(w)
    if kern == "decode_f8f4_kernel":
        return (f"u{w.bits} codes as the fp4 operand; dequantized query as 4 fp8 digits "
                "(about 16 bits of each value), probabilities as 16-bit fixed point per "
                "32-token block in 4 fp8 nibble digits; fp16 windows on f16 matrix cores; "
                "fp32 accumulate and softmax")
    if kern == "decode_mfma_kernel":
        return (f"u{w.bits} codes as subnormal fp16 operands; query / probabilities as fp16 "
                "hi+lo (about 22 bits); fp32 accumulate and softmax")
    return f"u{w.bits} codes, fp32 vector-ALU math"


def split_append(w, n_chunks: int) -> bool:
    """Whether the split-K launch also quantizes the appended group (the
    library's dispatch rule: the 2-bit matrix-core kernel with plain codes and
    at least 4 chunks, or with the 16-channel Kitty boost when it merges in
    place, or the 4-bit matrix-core kernel)."""
    kern = split_kernel(w)
    if kern == "decode_f8f4_kernel":
        return n_chunks >= 4 if w.n_boost == 0 else in_launch_merge(w, n_chunks)
    return kern == "decode_mfma_kernel"


def per_wave_chunks(w, n_chunks: int) -> bool:
    """Whether the 2-bit kernel runs one chunk per consumer wave (plain codes,
    GQA 4, a multiple of 8 chunks, at least 32, and at least 256 blocks of 8
    chunks over all heads): its parts are then blocks of 8 chunks."""
    return (split_kernel(w) == "decode_f8f4_kernel" and w.n_boost == 0 and w.gqa == 4
            and n_chunks % 8 == 0 and n_chunks >= 32 and (n_chunks // 8) * w.heads >= 256)


def in_launch_merge(w, n_chunks: int) -> bool:
    """Whether the split-K launch merges its parts in place (matrix-core
    kernels: at most 8 parts, or 32 blocks of 8 chunks)."""
    if split_kernel(w) == "decode_valu_kernel":
        return False
    if per_wave_chunks(w, n_chunks):
        return n_chunks // 8 <= 32
    return n_chunks <= 8


def fused_step(w, n_chunks: int) -> bool:
    """Whether the library runs a step with append as one launch (split-K with
    the append, and the merge in the same launch)."""
    return split_append(w, n_chunks) and in_launch_merge(w, n_chunks)


def launches_per_step(w, n_chunks: int, append: bool) -> int:
    """Kernel launches of one kvq_decode_step call (the library's dispatch)."""
    mfma = split_kernel(w) != "decode_valu_kernel"
    n_parts = (n_chunks // 8 if per_wave_chunks(w, n_chunks) else n_chunks) if mfma \
        else n_chunks + 1
    merged = in_launch_merge(w, n_chunks)
    if append:
        if split_append(w, n_chunks):
            return 1 if merged else 2
        return 2 if n_parts <= 32 else 3
    return 1 if merged else 2


def kernel_source_hash() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bit_kv_cache_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mx_kernel(w) -> str:
    """Kernel name (with template arguments, as the profiler prints it) of the
    MXFP4 decode for this workload."""
    if w.gqa in (4, 8) and w.T % 128 == 0:
        return f"decode_f8f4_kernel<{w.gqa}, false, true, false>"
    return "decode_mx_kernel"


def traffic_file(w, mx: bool = False) -> str:
    kern = "decode_f8f4_kernel_mxfp4" if mx else split_kernel(w)
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{kern}_{w.name}.txt")


# kernels of the library (and the copy kernel) whose counters are recorded
TRAFFIC_KERNELS = ("decode_", "merge_", "quantize_kernel", "mx_quantize_kernel")


def _counter_means(csv_path, counter):
    """Mean counter value per dispatch of every library kernel in the run, by
    the kernel's name with template arguments."""
    import csv
    import re
    per = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if COPY_KERNEL in name:
                key = COPY_KERNEL
            else:
                m = re.search(r"(\w+_kernel)(<[^()]*>)?\(", name)
                if not m or not m.group(1).startswith(TRAFFIC_KERNELS):
                    continue
                key = m.group(1) + (m.group(2) or "")
            per.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def write_traffic(w, fetch_csv: str, write_csv: str, command: str, mx: bool = False) -> dict:
    """Turn the two counter runs into bytes per launch of the decode kernel
    (and of every other library kernel the run launched)."""
    want = mx_kernel(w) if mx else split_kernel(w)
    fm, fn = _counter_means(fetch_csv, "FETCH_SIZE")
    wm, wn = _counter_means(write_csv, "WRITE_SIZE")
    f_scale = CALIB_COPY_BYTES / (fm[COPY_KERNEL] * 1024)
    w_scale = CALIB_COPY_BYTES / (wm[COPY_KERNEL] * 1024)
    # the decode kernel: the most-launched instantiation matching its name
    kern = max((k for k in fm if k.startswith(want) or want.startswith(k)),
               key=lambda k: fn[k])
    fetch = fm[kern] * 1024 * f_scale
    write = wm[kern] * 1024 * w_scale
    others = {k: {"fetch_bytes": round(fm[k] * 1024 * f_scale),
                  "write_bytes": round(wm.get(k, 0.0) * 1024 * w_scale),
                  "dispatches": fn[k]}
              for k in sorted(fm) if k not in (kern, COPY_KERNEL)}
    rec = {"workload": w.name + ("_mxfp4" if mx else ""), "kernel": kern,
           "source_hash": kernel_source_hash(),
           "fetch_bytes": round(fetch), "write_bytes": round(write),
           "traffic_bytes": round(fetch + write),
           "raw_fetch_kib": round(fm[kern], 1), "raw_write_kib": round(wm[kern], 1),
           "copy_fetch_kib": round(fm[COPY_KERNEL], 1), "copy_write_kib": round(wm[COPY_KERNEL], 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "dispatches": {"fetch": fn, "write": wn}, "other_kernels": others}
    with open(traffic_file(w, mx), "w") as fh:
        fh.write(f"# HBM traffic per launch of {kern}, workload {w.name}\n")
        fh.write(f"# counters: {command}\n")
        fh.write(f"# scale = {CALIB_COPY_BYTES} B copied / counter reading of the copy kernel\n")
        for k, v in rec.items():
            fh.write(f"{k}: {json.dumps(v)}\n")
    return rec


def read_traffic(w, mx: bool = False):
    """Bytes per launch from the committed counter file, or None when absent or
    taken from other kernel sources."""
    try:
        rec = {}
        with open(traffic_file(w, mx)) as fh:
            for ln in fh:
                if ln.startswith("#") or ":" not in ln:
                    continue
                k, v = ln.split(":", 1)
                rec[k.strip()] = json.loads(v)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes")


def _host_info():
    cores = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = cores
    model = platform.processor() or "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=5).stdout
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                model = ln.split(":", 1)[1].strip()
    except Exception:
        pass
    try:   # the kernel's own name for the part, when lscpu's is generic
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    name = ln.split(":", 1)[1].strip()
                    if len(name) > len(model):
                        model = name
                    break
    except OSError:
        pass
    return min(cores, aff), model


def build_caches(w, n_copies, kvq, synth, torch):
    cfg = kvq.QCfg(bits=w.bits, group=w.G, head_dim=w.D, n_boost=w.n_boost)
    t_cap = w.T + w.G
    c0 = kvq.Cache.empty(cfg, w.heads, t_cap)
    hb = max(1, min(w.heads, (1 << 30) // max(1, w.T * w.D * 4)))  # ~1 GiB of source per batch
    for h0 in range(0, w.heads, hb):
        n = min(hb, w.heads - h0)
        ks, vs = zip(*[synth.head_kv(w, h, "cuda") for h in range(h0, h0 + n)])
        k, v = torch.stack(ks), torch.stack(vs)
        kvq.kvq_quantize_pack(cfg, c0.heads_view(h0, n), 1, n, k, v, 0, w.T // w.G)
        del k, v, ks, vs
    torch.cuda.synchronize()
    copies = [c0]
    for _ in range(n_copies - 1):
        copies.append(kvq.Cache(cfg, t_cap, w.heads,
                                **{f: (None if getattr(c0, f) is None else getattr(c0, f).clone())
                                   for f in kvq.Cache.FIELDS}))
    torch.cuda.synchronize()
    return cfg, copies


def cpu_baseline(w, max_heads, threads, one_thread_heads=4, reps=3):
    """Time the oracle (as it stands) on bounded samples of the workload, each
    figure the median of ``reps`` runs scaled to all kv heads:
      * one decode step (attention over the whole cache and windows, plus the
        quantize of the appended group) on all ``threads`` host threads over
        up to ``max_heads`` kv heads, and on one thread over
        ``one_thread_heads`` kv heads;
      * quantize-all (the whole T-token cache) on the same two samples.
    The headline ``value`` is the all-threads step."""
    import numpy as np
    import oracle
    import synth

    def sample(n_heads):
        heads = list(range(min(n_heads, w.heads)))
        if len(heads) >= w.H_kv:
            heads = heads[: (len(heads) // w.H_kv) * w.H_kv]
        B = max(1, len(heads) // w.H_kv)
        H_kv = min(w.H_kv, len(heads))
        ks, vs, kr, vr, kS, vS = [], [], [], [], [], []
        for h in heads:
            k, v = synth.head_kv(w, h, "cpu")
            a, b, c, d = synth.head_windows(w, h, "cpu")
            ks.append(synth.as_bits(k)), vs.append(synth.as_bits(v))
            kS.append(synth.as_bits(a)), vS.append(synth.as_bits(b))
            kr.append(synth.as_bits(c)), vr.append(synth.as_bits(d))
        q = synth.as_bits(synth.query(w, "cpu"))[:B, : H_kv * w.gqa]
        return (heads, B, H_kv, np.stack(ks), np.stack(vs), q,
                *(np.stack(x) for x in (kS, vS, kr, vr)))

    def run(n_heads, n_threads):
        heads, B, H_kv, k_src, v_src, q, kS, vS, kr, vr = sample(n_heads)
        oc = oracle.empty_cache(w.bits, w.G, w.D, w.n_boost, w.T + w.G, len(heads))
        quant, step = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.quantize_pack(oc, k_src, v_src, 0, w.T // w.G, n_threads=n_threads)
            quant.append(time.perf_counter() - t0)
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.decode_attention(oc, B, H_kv * w.gqa, H_kv, q, w.T,
                                    k_sink=kS if w.S else None, v_sink=vS if w.S else None,
                                    n_sink=w.S, k_res=kr, v_res=vr, n_res=w.R,
                                    n_threads=n_threads)
            if w.R >= w.G:
                oracle.quantize_pack(oc, kr, vr, w.T // w.G, 1, n_threads=n_threads)
            step.append(time.perf_counter() - t0)
        scale = w.heads / len(heads)
        us = lambda xs: sorted(round(x * scale * 1e6, 1) for x in xs)
        return len(heads), us(step), us(quant)

    n_all, step_all, quant_all = run(max_heads, threads)
    n_one, step_one, quant_one = run(one_thread_heads, 1)
    med = lambda xs: xs[len(xs) // 2]
    return {"value": med(step_all), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"one decode step (attention + append quantize) over {n_all} of {w.heads} "
                      f"kv heads on {threads} threads, median of {reps}, scaled x"
                      f"{w.heads / n_all:g}",
            "one_thread": {"value": med(step_one), "unit": "us/step", "cores": 1,
                           "runs": step_one,
                           "sample": f"{n_one} of {w.heads} kv heads, median of {reps}, scaled "
                                     f"x{w.heads / n_one:g}"},
            "all_threads_runs": step_all,
            "quantize_all": {"unit": "us per whole-cache quantize (T tokens, all kv heads)",
                             "all_threads": med(quant_all), "all_threads_runs": quant_all,
                             "one_thread": med(quant_one), "one_thread_runs": quant_one}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (about 20 ms: the clocks reach their steady state)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0 = auto)")
    ap.add_argument("--n-chunks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=1 << 20, help="kv heads the oracle runs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the run, stream 1 GiB in and 1 GiB out 5 times (counter scale)")
    ap.add_argument("--profile-step", action="store_true",
                    help="launch only the warm-up and timed steps (counter runs), then exit")
    ap.add_argument("--mxfp4", action="store_true",
                    help="time the MXFP4 cache's decode (kvq_mx_decode_attention) on the "
                         "workload's shape instead")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "CMD"),
                    help="write the profiles/ traffic file from two counter runs and exit")
    args = ap.parse_args(argv)

    if args.write_traffic:
        import synth
        print(json.dumps(write_traffic(synth.WORKLOADS[args.workload], *args.write_traffic,
                                       mx=args.mxfp4)))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (each box has "
              "one GPU and the path is built for a single device).", file=sys.stderr)
        return 2

    import torch

    import bit_kv_cache_amd as kvq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.mxfp4:
        return bench_mx(args, w, torch, kvq, synth)
    cache_bytes_one = None

    # packed caches (rotated) -----------------------------------------------------
    probe_cfg = kvq.QCfg(bits=w.bits, group=w.G, head_dim=w.D, n_boost=w.n_boost)
    one = kvq.Cache.empty(probe_cfg, 1, w.T + w.G, device="meta").nbytes() * w.heads
    cache_bytes_one = one
    n_copies = args.copies or max(2, math.ceil(3 * MALL_BYTES / one) + 1)
    n_copies = min(n_copies, 16)
    cfg, copies = build_caches(w, n_copies, kvq, synth, torch)

    # windows and query -------------------------------------------------------------
    wins = [synth.head_windows(w, h, "cuda") for h in range(w.heads)]
    k_sink = torch.stack([x[0] for x in wins])
    v_sink = torch.stack([x[1] for x in wins])
    k_res = torch.stack([x[2] for x in wins])
    v_res = torch.stack([x[3] for x in wins])
    del wins
    q = synth.query(w, "cuda")
    n_chunks, ws_bytes = kvq.kvq_decode_plan(cfg, w.B, w.H_q, w.H_kv, w.T,
                                             args.n_chunks or w.min_chunks)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((w.B, w.H_q, w.D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # raw ctypes arguments, built once (keeps host launch overhead low)
    lib = kvq._lib
    c_cfg = cfg.c()
    c_caches = [c.c() for c in copies]
    sink = kvq.window(k_sink, v_sink, w.S)
    res = kvq.window(k_res, v_res, w.R)
    sink_p = ctypes.byref(sink) if sink is not None else None
    res_p = ctypes.byref(res) if res is not None else None
    append = w.R >= w.G
    g_app = w.T // w.G

    n_parts = ctypes.c_int32(0)

    def partials(i):
        st = lib.kvq_decode_partials(ctypes.byref(c_cfg), ctypes.byref(c_caches[i % n_copies]),
                                     w.B, w.H_q, w.H_kv, q.data_ptr(), w.T, sink_p, res_p,
                                     ctypes.c_float(0.0), n_chunks, ws.data_ptr(), ws_bytes,
                                     ctypes.byref(n_parts), sp)
        if st:
            raise kvq.KvqError(st, "kvq_decode_partials")

    def merge():
        st = lib.kvq_decode_merge(w.B, w.H_q, n_parts.value, ws.data_ptr(), ws_bytes,
                                  out.data_ptr(), sp)
        if st:
            raise kvq.KvqError(st, "kvq_decode_merge")

    def decode(i):
        partials(i)
        merge()

    def quant(i):
        if not append:
            return
        st = lib.kvq_quantize_pack(ctypes.byref(c_cfg), ctypes.byref(c_caches[i % n_copies]),
                                   1, w.heads, k_res.data_ptr(), v_res.data_ptr(),
                                   k_res.stride(0), g_app, 1, sp)
        if st:
            raise kvq.KvqError(st, "kvq_quantize_pack")

    def step(i):
        # one whole step: decode + append of the full residual group, one call
        # (the append runs inside the split-K launch where the path fuses it)
        st = lib.kvq_decode_step(ctypes.byref(c_cfg), ctypes.byref(c_caches[i % n_copies]),
                                 w.B, w.H_q, w.H_kv, q.data_ptr(), w.T, sink_p, res_p,
                                 ctypes.c_float(0.0), n_chunks, ws.data_ptr(), ws_bytes,
                                 out.data_ptr(), 1 if append else 0, sp)
        if st:
            raise kvq.KvqError(st, "kvq_decode_step")

    # The plain read of the split-K phase's bytes (the reference rate reported
    # beside the roofline) runs before the warm-up: its ~0.1 s of streaming
    # also brings the clocks to their steady state, which a few warm-up steps
    # alone do not.  It leaves its own buffers, not the caches, in the MALL.
    sr = None
    if not args.profile_step:
        sr = stream_read_ceiling(kvq, torch, decode_bytes(w) - w.B * w.H_q * w.D * 4, n_copies,
                                 stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: whole steps -------------------------------------------------------
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    if args.profile_step:
        print(json.dumps({"profile_step": w.name, "steps": args.steps,
                          "ms_per_step": round(ms_per_step, 5)}), flush=True)
        if args.calib_copy:
            calib_copy(torch)
        return 0

    # the same step as three launches (decode partials, merge, quantize), for context
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        decode(i)
        quant(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = e0.elapsed_time(e1) / args.steps

    # per-kernel durations on the launch stream (HIP events between the launches)
    n_k = min(args.steps, 100)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_k)]
    torch.cuda.synchronize()
    for i in range(n_k):
        ev[i][0].record(stream)
        partials(i)
        ev[i][1].record(stream)
        merge()
        ev[i][2].record(stream)
        quant(i)
        ev[i][3].record(stream)
    torch.cuda.synchronize()

    def stats(a, b):
        ms = sorted(e[a].elapsed_time(e[b]) for e in ev)
        return sum(ms) / n_k, ms

    part_iso, part_ms = stats(0, 1)
    merge_iso, _ = stats(1, 2)
    dec_avg, dec_ms = stats(0, 2)

    # average launch duration of each kernel alone, back to back on the
    # stream (one event pair around n_k launches: no event between launches)
    def back_to_back(fn):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for i in range(n_k):
            fn(i)
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / n_k

    def attention(i):
        st = lib.kvq_decode_step(ctypes.byref(c_cfg), ctypes.byref(c_caches[i % n_copies]),
                                 w.B, w.H_q, w.H_kv, q.data_ptr(), w.T, sink_p, res_p,
                                 ctypes.c_float(0.0), n_chunks, ws.data_ptr(), ws_bytes,
                                 out.data_ptr(), 0, sp)
        if st:
            raise kvq.KvqError(st, "kvq_decode_step")

    # three interleaved rounds of each, the median of each kept (one pass in a
    # fixed order let the figure measured right after a long run of another
    # launch read a few microseconds high)
    legs = [("step", step), ("attention", attention), ("partials", partials),
            ("merge", lambda i: merge())] + ([("quant", quant)] if append else [])
    runs = {name: [] for name, _ in legs}
    for _ in range(3):
        for name, fn in legs:
            runs[name].append(back_to_back(fn))
    med = {name: sorted(v)[1] for name, v in runs.items()}
    step_avg, attn_avg, part_avg, merge_avg = (med["step"], med["attention"], med["partials"],
                                               med["merge"])
    app_avg = med["quant"] if append else 0.0

    alg = decode_bytes(w)
    alg_split = alg - w.B * w.H_q * w.D * 4   # the split-K phase does not write O
    step_bytes = alg + (append_bytes(w) if append else 0)
    eff_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    one_launch = append and fused_step(w, n_chunks)
    split_gbps = alg_split / (part_avg * 1e-3) / 1e9
    if one_launch:
        # the step is one launch of the split-K kernel that also quantizes the
        # appended group and merges: its bytes are the whole step's
        dom_kernel = f"{split_kernel(w)} (whole step in one launch: split-K, append, merge)"
        dom_bytes, dom_avg = step_bytes, step_avg
    else:
        dom_kernel = f"{split_kernel(w)} (split-K phase, kvq_decode_partials)"
        dom_bytes, dom_avg = alg_split, part_avg
    achieved = dom_bytes / (dom_avg * 1e-3) / 1e9

    result = {
        "metric": "decode-attn us/step + effective HBM GB/s (% of peak), 2-bit, Llama-3-8B "
                  "shape 32K" if w.name == DEFAULT_WORKLOAD else f"decode-attn us/step ({w.name})",
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(w),
        "data": "synthetic (seeded; K outlier channels, see synth/)",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "D": w.D,
                   "T": w.T, "R": w.R, "S": w.S, "bits": w.bits, "G": w.G,
                   "n_boost": w.n_boost, "n_chunks": n_chunks, "cache_copies": n_copies,
                   "cache_bytes_per_copy": cache_bytes_one, "step": "decode + append-group "
                   "quantize (kvq_decode_step)" if append else "decode (kvq_decode_step)",
                   "launches_per_step": launches_per_step(w, n_chunks, append)},
        "effective_GBps": round(eff_gbps, 1),
        "effective_frac_of_peak": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "step_bytes": step_bytes,
        "decode_us": {"step_avg": round(step_avg * 1e3, 3),
                      "step_without_append_avg": round(attn_avg * 1e3, 3),
                      "split_kernel_avg": round(part_avg * 1e3, 3),
                      "merge_kernel_avg": round(merge_avg * 1e3, 3),
                      "split_plus_merge_isolated_avg": round(dec_avg * 1e3, 3),
                      "split_plus_merge_p10": round(dec_ms[n_k // 10] * 1e3, 3),
                      "split_plus_merge_p90": round(dec_ms[(9 * n_k) // 10] * 1e3, 3),
                      "split_kernel_isolated_avg": round(part_iso * 1e3, 3),
                      "merge_kernel_isolated_avg": round(merge_iso * 1e3, 3),
                      "timing": "*_avg: n launches back to back between two HIP events on the "
                                "launch stream, the median of three interleaved rounds; "
                                "*_isolated_*: an event pair around every launch"},
        "append_quant_us": round(app_avg * 1e3, 3) if append else None,
        "step_as_three_launches_us": round(ms_unfused * 1e3, 3),
        "split_phase": {"kernel": f"{split_kernel(w)} (kvq_decode_partials)",
                        "algorithmic_bytes": alg_split, "avg_us": round(part_avg * 1e3, 3),
                        "GBps": round(split_gbps, 1),
                        "frac": round(split_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": read_traffic(w),
                     "kernel": dom_kernel,
                     "algorithmic_bytes": dom_bytes,
                     "kernel_avg_us": round(dom_avg * 1e3, 3)},
    }
    result["stream_read"] = sr
    result["roofline"]["frac_of_stream_read"] = round(achieved / sr["GBps"], 4)
    if not args.no_cpu_baseline:
        cores, model = _host_info()
        cb = cpu_baseline(w, args.cpu_heads, cores)
        cb["cpu_model"] = model
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    if args.calib_copy:
        calib_copy(torch)
    return 0


def stream_read_ceiling(kvq, torch, nbytes, n_copies, stream, reps=50):
    """The bandwidth a plain read reaches over the same bytes as the split-K
    phase, rotating over as many independent copies as the caches: the best
    of a sweep over grid size, workgroup size and load kind."""
    nbytes = (nbytes + 15) // 16 * 16
    bufs = [torch.full((nbytes // 4,), i, dtype=torch.int32, device="cuda")
            for i in range(n_copies)]
    sink = torch.zeros(8192 * 1024, dtype=torch.int32, device="cuda")
    best = None
    for mode in (0, 1):
        for threads in (256, 512, 1024):
            for blocks in (256, 512, 1024, 2048, 4096, 8192):
                run = lambda i: kvq.kvq_stream_read(bufs[i % n_copies], sink, blocks, threads,
                                                    mode, stream=stream)
                for i in range(2 * n_copies):
                    run(i)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for i in range(reps):
                    run(i)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / reps * 1e3
                if best is None or us < best[0]:
                    best = (us, blocks, threads, mode)
    us, blocks, threads, mode = best
    gbps = nbytes / (us * 1e-6) / 1e9
    del bufs, sink
    return {"kernel": "stream_read_kernel (kvq_stream_read)", "bytes": nbytes,
            "avg_us": round(us, 3), "GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "best_config": {"blocks": blocks, "threads": threads,
                            "loads": "non-temporal" if mode else "ordinary"},
            "sweep": "blocks 256..8192 x threads 256/512/1024 x ordinary/non-temporal loads, "
                     f"{reps} launches back to back per point"}


def bench_mx(args, w, torch, kvq, synth):
    """Decode over an MXFP4 cache of the workload's shape (32-value blocks,
    E8M0 scales, E2M1 values), its keys and values from the same seeded
    generator; one JSON line."""
    D, T, heads = w.D, w.T, w.heads
    per_head = T * (D // 8 * 4 + D // 32) * 2          # codes + scales, K and V
    n_copies = min(16, args.copies or max(2, math.ceil(3 * MALL_BYTES / (per_head * heads)) + 1))
    copies = [kvq.MxCache.empty(heads, T) for _ in range(n_copies)]
    for h in range(heads):
        k, v = synth.head_kv(w, h, "cuda")
        for c in copies:
            one = kvq.MxCache(T, 1, c.k_codes[h:h + 1], c.k_scale[h:h + 1], c.v_codes[h:h + 1],
                              c.v_scale[h:h + 1])
            kvq.kvq_mx_quantize_pack(one, 1, 1, k[None], v[None], 0, T)
        del k, v
    wins = [synth.head_windows(w, h, "cuda") for h in range(heads)]
    k_res = torch.stack([x[2] for x in wins])
    v_res = torch.stack([x[3] for x in wins])
    res = kvq.window(k_res, v_res, w.R)
    sink = None
    if w.S:
        sink = kvq.window(torch.stack([x[0] for x in wins]), torch.stack([x[1] for x in wins]), w.S)
    q = synth.query(w, "cuda")
    n_chunks, ws_bytes = kvq.kvq_mx_decode_plan(w.B, w.H_q, w.H_kv, T, args.n_chunks)
    ws = kvq.decode_workspace(ws_bytes)
    out = torch.empty((w.B, w.H_q, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        kvq.kvq_mx_decode_attention(copies[i % n_copies], w.B, w.H_q, w.H_kv, q, T, sink, res,
                                    out, ws, n_chunks=n_chunks, stream=stream)

    n_win = w.S + w.R
    alg = heads * per_head + heads * n_win * D * 2 * 2 + w.B * w.H_q * D * (2 + 4)
    # the plain-read reference first: it also brings the clocks to their
    # steady state before the warm-up (as in the min-max bench)
    sr = None if args.profile_step else stream_read_ceiling(kvq, torch, alg, n_copies, stream)
    for i in range(args.warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    if args.profile_step:
        print(json.dumps({"profile_step": w.name + "_mxfp4", "steps": args.steps,
                          "us_per_step": round(us, 3)}), flush=True)
        if args.calib_copy:
            calib_copy(torch)
        return 0
    gqa = w.H_q // w.H_kv
    if gqa in (4, 8) and T % 128 == 0:   # the block-scaled matrix-core kernel
        kern = f"decode_f8f4_kernel<{gqa},mxfp4> (kvq_mx_decode_attention, " + (
            "one launch, in-launch merge)" if n_chunks <= 8 else "+ merge launch)")
    else:
        kern = "decode_mx_kernel + merge (kvq_mx_decode_attention, two launches)"
    gbps = alg / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": f"decode-attn us/step ({w.name} shape, MXFP4 cache)", "value": round(us, 3),
        "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e2m1 codes with e8m0 block scales as the fp4 operand; query and "
                  "probabilities as 4 fp8 digits (about 16 bits); fp16 windows on f16 "
                  "matrix cores; fp32 accumulate and softmax"
                  if gqa in (4, 8) and T % 128 == 0 else
                  "e2m1 codes with e8m0 block scales, fp32 vector-ALU math"),
        "data": "synthetic (seeded; the workload's generator)",
        "config": {"workload": f"{w.name}_mxfp4", "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "D": D, "T": T, "R": w.R, "S": w.S, "block": 32, "n_chunks": n_chunks,
                   "cache_copies": n_copies, "step": "decode (kvq_mx_decode_attention)"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": read_traffic(w, mx=True),
                     "kernel": kern,
                     "algorithmic_bytes": alg, "kernel_avg_us": round(us, 3),
                     "frac_of_stream_read": round(gbps / sr["GBps"], 4)},
        "stream_read": sr}), flush=True)
    return 0


def calib_copy(torch):
    """1 GiB in and 1 GiB out, 5 times: the reference the traffic counters are
    scaled by."""
    src = torch.zeros(CALIB_COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


if __name__ == "__main__":
    sys.exit(main())
