"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/kvq.h declares, and rejects bad arguments before launching
anything (only calls that must fail validation are made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

kvq = pytest.importorskip("bit_kv_cache_amd")


def _declared():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _declared()
    assert names == sorted(kvq.EXPORTED)
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_header_workspace_constants_match_binding():
    """The binding's workspace offsets are the header's: the status words sit
    after the 65536 arrival counters and inside the counter bytes."""
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    consts = {m.group(1): int(m.group(2))
              for m in re.finditer(r"#define\s+(KVQ_WS_[A-Z_]+)\s+(\d+)", src)}
    assert consts["KVQ_WS_COUNTER_BYTES"] == kvq.KVQ_WS_COUNTER_BYTES
    assert consts["KVQ_WS_STATUS"] == kvq.KVQ_WS_STATUS == 65536 * 4
    assert kvq.KVQ_WS_STATUS + 8 <= kvq.KVQ_WS_COUNTER_BYTES
    assert kvq.KVQ_WS_COUNTER_BYTES % 16 == 0   # the records stay 16-byte aligned
    m = re.search(r"#define\s+KVQ_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kvq.KVQ_NOALLOC_SCRATCH_BYTES


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert kvq.kvq_status_string(s).startswith("KVQ_")
    assert "unknown" in kvq.kvq_status_string(7)


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _cfg(bits=2, group=128, D=128, nb=0, vb=0, score=0):
    return kvq.kvq_qcfg(bits, group, D, nb, vb, score)


def _cache(t_cap=1024, align=0, hi=FAKE):
    p = FAKE + align
    return kvq.kvq_cache(p, p, p, hi, hi, p, p, p, t_cap, None, 0)


def _quant(cfg, cache, B=1, H=1, k=FAKE, v=FAKE, stride=128 * 128, fg=0, ng=1):
    return kvq.raw_call("kvq_quantize_pack", ctypes.byref(cfg) if cfg else None,
                        ctypes.byref(cache) if cache else None, B, H, k, v, stride, fg, ng, None)


@pytest.mark.parametrize("cfg,want", [
    (_cfg(bits=3), kvq.KVQ_ERR_ARG),
    (_cfg(bits=1), kvq.KVQ_ERR_ARG),
    (_cfg(bits=8, nb=16), kvq.KVQ_ERR_ARG),        # the boost is for 2-bit codes
    (_cfg(vb=3), kvq.KVQ_ERR_ARG),
    (_cfg(nb=16, vb=4), kvq.KVQ_ERR_ARG),          # Kitty values are 2-bit
    (_cfg(score=2), kvq.KVQ_ERR_ARG),
    (_cfg(vb=8), kvq.KVQ_ERR_UNSUPPORTED),         # mixed widths built: K2V4, K4V2
    (_cfg(bits=4, vb=8), kvq.KVQ_ERR_UNSUPPORTED),
    (_cfg(group=64, vb=4), kvq.KVQ_ERR_UNSUPPORTED),   # mixed widths: G = 128 only
    (_cfg(D=64), kvq.KVQ_ERR_UNSUPPORTED),
    (_cfg(group=48), kvq.KVQ_ERR_ARG),
    (_cfg(group=8), kvq.KVQ_ERR_ARG),
    (_cfg(group=0), kvq.KVQ_ERR_ARG),
    (_cfg(nb=8), kvq.KVQ_ERR_ARG),
    (_cfg(bits=4, nb=16), kvq.KVQ_ERR_ARG),
    (_cfg(nb=144), kvq.KVQ_ERR_ARG),
])
def test_quantize_rejects_bad_config(cfg, want):
    assert _quant(cfg, _cache()) == want


def test_paged_cache_validation():
    """A page table needs a positive row stride, 4-byte alignment, and rows long
    enough for every group a call touches (checked before any launch)."""
    cfg = _cfg()
    def paged(stride, table=FAKE, t_cap=1024):
        return kvq.kvq_cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t_cap, table, stride)
    assert _quant(cfg, paged(0)) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, paged(-4)) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, paged(8, table=FAKE + 2)) == kvq.KVQ_ERR_ALIGN
    assert _quant(cfg, paged(4), fg=3, ng=2) == kvq.KVQ_ERR_ARG      # group 4 past the rows
    # the pool size (t_cap) does not bound group indices in a paged cache
    assert _quant(cfg, paged(64, t_cap=256), fg=40, ng=1, k=None) == kvq.KVQ_ERR_ARG  # k checked
    # decode: the quantized groups must fit the rows
    assert _decode(cache=paged(4), nq=5 * 128) == kvq.KVQ_ERR_ARG


def test_ragged_decode_validation():
    """The per-sequence length arrays must be 4-byte aligned; everything else is
    validated as in the uniform call (nothing is launched on an error)."""
    def rag(sq=None, sr=None, out=FAKE, Hq=4):
        cfg, cache = _cfg(), _cache()
        return kvq.raw_call("kvq_decode_attention_ragged", ctypes.byref(cfg), ctypes.byref(cache),
                            1, Hq, 1, FAKE, 1024, None, None, sq, sr, ctypes.c_float(0.0), 0,
                            FAKE, 1 << 30, out, None)
    assert rag(sq=FAKE + 2) == kvq.KVQ_ERR_ALIGN
    assert rag(sr=FAKE + 1) == kvq.KVQ_ERR_ALIGN
    assert rag(out=None) == kvq.KVQ_ERR_ARG
    assert rag(Hq=6) == kvq.KVQ_ERR_UNSUPPORTED     # a GQA group of 6 is not built


def test_quantize_rejects_bad_arguments():
    cfg = _cfg()
    assert _quant(None, _cache()) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, None) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, _cache(t_cap=100)) == kvq.KVQ_ERR_ARG        # not a multiple of G
    assert _quant(cfg, _cache(align=4)) == kvq.KVQ_ERR_ALIGN
    assert _quant(cfg, _cache(), B=0) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, _cache(), fg=-1) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, _cache(t_cap=256), fg=1, ng=2) == kvq.KVQ_ERR_ARG   # past t_cap
    assert _quant(cfg, _cache(), k=None) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, _cache(), stride=100) == kvq.KVQ_ERR_ARG
    assert _quant(cfg, _cache(), k=FAKE + 2) == kvq.KVQ_ERR_ALIGN
    assert _quant(_cfg(nb=16), _cache(hi=None)) == kvq.KVQ_ERR_ARG


def test_quantize_zero_groups_is_noop():
    assert _quant(_cfg(), _cache(), ng=0) == kvq.KVQ_OK


def _decode(cfg=None, cache=None, B=1, Hq=4, Hkv=1, q=FAKE, nq=1024, sink=None, res=None,
            nchunks=0, ws=FAKE, ws_bytes=1 << 30, out=FAKE):
    cfg = cfg or _cfg()
    cache = cache or _cache()
    return kvq.raw_call("kvq_decode_attention", ctypes.byref(cfg), ctypes.byref(cache), B, Hq,
                        Hkv, q, nq, ctypes.byref(sink) if sink else None,
                        ctypes.byref(res) if res else None, ctypes.c_float(0.0), nchunks, ws,
                        ws_bytes, out, None)


def test_decode_rejects_bad_arguments():
    assert _decode(Hq=6, Hkv=4) == kvq.KVQ_ERR_ARG            # H_q not a multiple of H_kv
    assert _decode(Hq=16, Hkv=1) == kvq.KVQ_ERR_UNSUPPORTED   # group of 16 query heads
    assert _decode(Hq=3, Hkv=1) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(nq=100) == kvq.KVQ_ERR_ARG                 # not a multiple of G
    assert _decode(nq=2048) == kvq.KVQ_ERR_ARG                # past t_cap
    assert _decode(nq=-128) == kvq.KVQ_ERR_ARG
    assert _decode(nchunks=-1) == kvq.KVQ_ERR_ARG
    assert _decode(q=None) == kvq.KVQ_ERR_ARG
    assert _decode(out=FAKE + 8) == kvq.KVQ_ERR_ALIGN
    assert _decode(ws=None) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(ws_bytes=16) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(res=kvq.kvq_window(FAKE, FAKE, 5, 4)) == kvq.KVQ_ERR_ARG    # n > cap
    assert _decode(res=kvq.kvq_window(None, FAKE, 5, 8)) == kvq.KVQ_ERR_ARG
    assert _decode(sink=kvq.kvq_window(FAKE + 2, FAKE, 1, 8)) == kvq.KVQ_ERR_ALIGN


def test_decode_plan():
    cfg = kvq.QCfg(bits=2, group=128)
    # matrix-core path (GQA 4/8, G 128): resident blocks over the heads -- one
    # 8-wave block per CU for 2-bit codes, two 4-wave blocks per CU for 4-bit
    assert kvq.kvq_decode_plan(cfg, 8, 32, 8, 32768)[0] == 4
    assert kvq.kvq_decode_plan(cfg, 1, 32, 8, 1 << 20)[0] == 32
    assert kvq.kvq_decode_plan(cfg, 1, 32, 8, 1 << 20, 256)[0] == 256
    assert kvq.kvq_decode_plan(cfg, 32, 32, 8, 8192)[0] == 1
    assert kvq.kvq_decode_plan(cfg, 16, 64, 8, 131072)[0] == 2
    assert kvq.kvq_decode_plan(kvq.QCfg(bits=4, group=128), 32, 32, 8, 8192)[0] == 2
    assert kvq.kvq_decode_plan(cfg, 1, 32, 8, 0)[0] == 1      # windows only: one chunk
    nc, ws = kvq.kvq_decode_plan(cfg, 8, 32, 8, 32768)
    assert ws >= 8 * 32 * nc * 130 * 4
    # vector-ALU path (MHA): ~1024 blocks, at most one chunk per group
    assert kvq.kvq_decode_plan(cfg, 1, 1, 1, 512)[0] == 4
    assert kvq.kvq_decode_plan(cfg, 1, 1, 1, 0)[0] == 0
    assert kvq.kvq_decode_plan(kvq.QCfg(bits=2, group=64), 8, 32, 8, 32768)[0] == 16
    assert kvq.kvq_decode_workspace_bytes(cfg, 8, 32, 8, 32768) == ws
    nc, ws = kvq.kvq_decode_plan(cfg, 1, 1, 1, 512)
    assert ws >= (nc + 1) * 130 * 4
    assert kvq.kvq_decode_workspace_bytes(kvq.QCfg(bits=3), 8, 32, 8, 32768) == 0


def test_merge_rejects_bad_arguments():
    m = lambda B=1, H=4, n=8, ws=FAKE, wsb=1 << 20, out=FAKE: kvq.raw_call(
        "kvq_decode_merge", B, H, n, ws, wsb, out, None)
    assert m(n=0) == kvq.KVQ_ERR_ARG
    assert m(n=1025) == kvq.KVQ_ERR_ARG
    assert m(B=0) == kvq.KVQ_ERR_ARG
    assert m(ws=None) == kvq.KVQ_ERR_WORKSPACE
    assert m(wsb=4 * 8 * 130 * 4 - 4) == kvq.KVQ_ERR_WORKSPACE
    assert m(out=None) == kvq.KVQ_ERR_ARG
    assert m(out=FAKE + 4) == kvq.KVQ_ERR_ALIGN


def test_partials_reject_bad_arguments():
    def p(n_parts=True, **kw):
        cfg, cache = _cfg(), _cache()
        nq = kw.get("nq", 1024)
        out = ctypes.c_int32(0)
        return kvq.raw_call("kvq_decode_partials", ctypes.byref(cfg), ctypes.byref(cache), 1, 4,
                            1, kw.get("q", FAKE), nq, None, None, ctypes.c_float(0.0), 0,
                            kw.get("ws", FAKE), 1 << 30,
                            ctypes.byref(out) if n_parts else None, None)
    assert p(n_parts=False) == kvq.KVQ_ERR_ARG
    assert p(nq=100) == kvq.KVQ_ERR_ARG
    assert p(q=FAKE + 2) == kvq.KVQ_ERR_ALIGN
    assert p(ws=None) == kvq.KVQ_ERR_WORKSPACE


@pytest.mark.parametrize("args,want", [
    ((None, 1024, FAKE, 256, 256, 0), kvq.KVQ_ERR_ARG),
    ((FAKE, 1024, None, 256, 256, 0), kvq.KVQ_ERR_ARG),
    ((FAKE + 4, 1024, FAKE, 256, 256, 0), kvq.KVQ_ERR_ALIGN),
    ((FAKE, 1000, FAKE, 256, 256, 0), kvq.KVQ_ERR_ALIGN),
    ((FAKE, 1024, FAKE, 256, 96, 0), kvq.KVQ_ERR_ARG),
    ((FAKE, 1024, FAKE, 256, 2048, 0), kvq.KVQ_ERR_ARG),
    ((FAKE, 1024, FAKE, 0, 256, 0), kvq.KVQ_ERR_ARG),
    ((FAKE, 1024, FAKE, (1 << 20) + 1, 256, 0), kvq.KVQ_ERR_ARG),
    ((FAKE, 1024, FAKE, 256, 256, 2), kvq.KVQ_ERR_ARG),
])
def test_stream_read_validation(args, want):
    assert kvq.raw_call("kvq_stream_read", *args, None) == want


def _mx(t_cap=1024, align=0):
    p = FAKE + align
    return kvq.kvq_mx_cache(p, p, p, p, t_cap)


@pytest.mark.parametrize("cache,args,want", [
    (None, (1, 1, FAKE, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ARG),
    (_mx(t_cap=1000), (1, 1, FAKE, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ARG),
    (_mx(align=4), (1, 1, FAKE, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ALIGN),
    (_mx(), (0, 1, FAKE, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ARG),
    (_mx(), (1, 1, FAKE, FAKE, 4096, 16, 32), kvq.KVQ_ERR_ARG),    # not a whole block
    (_mx(), (1, 1, FAKE, FAKE, 4096, 0, 48), kvq.KVQ_ERR_ARG),
    (_mx(), (1, 1, FAKE, FAKE, 4096, 1024, 32), kvq.KVQ_ERR_ARG),  # past t_cap
    (_mx(), (1, 1, None, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ARG),
    (_mx(), (1, 1, FAKE, FAKE, 100, 0, 32), kvq.KVQ_ERR_ARG),      # stride below n*D
    (_mx(), (1, 1, FAKE + 2, FAKE, 4096, 0, 32), kvq.KVQ_ERR_ALIGN),
])
def test_mx_quantize_validation(cache, args, want):
    c = ctypes.byref(cache) if cache is not None else None
    assert kvq.raw_call("kvq_mx_quantize_pack", c, *args, None) == want


def test_mx_dequantize_validation():
    c = _mx()
    assert kvq.raw_call("kvq_mx_dequantize", ctypes.byref(c), 1, 1, 1000, 32, FAKE, FAKE,
                        None) == kvq.KVQ_ERR_ARG
    assert kvq.raw_call("kvq_mx_dequantize", ctypes.byref(c), 1, 1, 0, 32, FAKE + 8, FAKE,
                        None) == kvq.KVQ_ERR_ALIGN


def test_mx_decode_plan_validation():
    def plan(*a):
        n, w = ctypes.c_int32(0), ctypes.c_size_t(0)
        return kvq.raw_call("kvq_mx_decode_plan", *a, ctypes.byref(n), ctypes.byref(w)), n.value
    assert plan(1, 32, 8, 512, 0)[0] == kvq.KVQ_OK
    assert plan(1, 32, 8, 500, 0)[0] == kvq.KVQ_ERR_ARG      # not whole 32-token blocks
    assert plan(1, 48, 8, 512, 0)[0] == kvq.KVQ_ERR_UNSUPPORTED
    assert plan(1, 30, 8, 512, 0)[0] == kvq.KVQ_ERR_ARG
    # at most one chunk per unit of work: a 128-token group on the matrix-core
    # path (GQA 4 / 8, whole groups), a 32-token block on the vector-ALU one
    assert plan(1, 32, 8, 512, 100)[1] == 4
    assert plan(1, 32, 8, 544, 100)[1] == 17
    assert plan(1, 8, 8, 512, 100)[1] == 16
    # automatic: one resident block per CU on the matrix-core path (256 / 64
    # heads), about 16 blocks per CU on the vector-ALU one
    assert plan(8, 32, 8, 32768, 0)[1] == 4
    assert plan(8, 64, 64, 32768, 0)[1] == 8
    c = _mx()
    assert kvq.raw_call("kvq_mx_decode_attention", ctypes.byref(c), 1, 32, 8, FAKE, 512, None,
                        None, ctypes.c_float(0.0), 0, FAKE, 16, FAKE, None) == kvq.KVQ_ERR_WORKSPACE


def test_noalloc_step_rejects_workspace_past_scratch():
    """kvq_decode_step_noalloc refuses a step whose workspace would exceed
    its scratch array (KVQ_ERR_WORKSPACE) before touching the GPU, and
    validates its arguments like kvq_decode_step."""
    def call(B, H_q, H_kv, T, n_chunks, cfg=None, cache=None, out=FAKE):
        cfg = cfg or _cfg()
        cache = cache or _cache(t_cap=1 << 20)
        return kvq.raw_call("kvq_decode_step_noalloc", ctypes.byref(cfg), ctypes.byref(cache),
                            B, H_q, H_kv, FAKE, T, None, None, ctypes.c_float(0.0), n_chunks,
                            out, 0, None)
    # 1024 x 64 query heads x 4 parts of (D + 2) floats: 136 MB > 8 MiB
    _, need = kvq.kvq_decode_plan(kvq.QCfg(bits=2, group=128), 1024, 64, 8, 4 * 128, 4)
    assert need > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert call(1024, 64, 8, 4 * 128, 4) == kvq.KVQ_ERR_WORKSPACE
    # 1 x 32 query heads x 256 parts fits (the 1M-token split)
    _, need = kvq.kvq_decode_plan(kvq.QCfg(bits=2, group=128), 1, 32, 8, 1 << 20, 256)
    assert need <= kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert call(1, 32, 8, 4 * 128, 4, cfg=_cfg(bits=3)) == kvq.KVQ_ERR_ARG
    assert call(1, 32, 8, 100, 4) == kvq.KVQ_ERR_ARG          # not a multiple of G
    assert call(1, 30, 8, 4 * 128, 4) == kvq.KVQ_ERR_ARG      # H_q % H_kv
