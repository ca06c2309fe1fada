"""Python binding of libkvq: low-bit KV cache + decode attention on MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvq.so`` (C ABI in ``include/kvq.h``).  torch provides device memory and
streams.  The functions keep the C names (``kvq_quantize_pack``,
``kvq_decode_attention``, ``kvq_dequantize``, ...) and take torch tensors;
a non-OK status raises ``KvqError``.  If the library is not built, importing
this package raises immediately -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB names another build of the same sources (the sanitizer test's
# host-instrumented one); there is no other implementation to fall back on
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libkvq.so is not built ({LIB_PATH}); run `python -m bit_kv_cache_amd._build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_ALIGN, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
# counter bytes at the start of a decode workspace: arrival counters (zero
# between calls), then the status words at KVQ_WS_STATUS
KVQ_WS_COUNTER_BYTES = 262400
KVQ_WS_STATUS = 262144

EXPORTED = ("kvq_status_string", "kvq_quantize_pack", "kvq_decode_plan",
            "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_step",
            "kvq_decode_partials", "kvq_decode_merge", "kvq_dequantize",
            "kvq_decode_attention_ragged", "kvq_decode_partials_ragged", "kvq_stream_read",
            "kvq_mx_quantize_pack", "kvq_mx_dequantize", "kvq_mx_decode_plan",
            "kvq_mx_decode_attention", "kvq_decode_step_noalloc")
# workspace bytes of the no-allocation decode step's scratch array (per GPU)
KVQ_NOALLOC_SCRATCH_BYTES = 8 << 20


class kvq_qcfg(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_boost", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("boost_score", ctypes.c_int32)]


class kvq_mx_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("t_cap", ctypes.c_int64)]


class kvq_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("k_min", ctypes.c_void_p), ("k_hi", ctypes.c_void_p),
                ("k_bidx", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("v_min", ctypes.c_void_p),
                ("t_cap", ctypes.c_int64), ("page_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int64)]


class kvq_window(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("cap", ctypes.c_int32)]


_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_lib.kvq_status_string.argtypes = [ctypes.c_int]
_lib.kvq_status_string.restype = ctypes.c_char_p
_lib.kvq_quantize_pack.argtypes = [_P, _P, _i32, _i32, _P, _P, _i64, _i64, _i64, _P]
_lib.kvq_quantize_pack.restype = ctypes.c_int
_lib.kvq_decode_plan.argtypes = [_P, _i32, _i32, _i32, _i64, _i32, _P, _P]
_lib.kvq_decode_plan.restype = ctypes.c_int
_lib.kvq_decode_workspace_bytes.argtypes = [_P, _i32, _i32, _i32, _i64, _i32]
_lib.kvq_decode_workspace_bytes.restype = _sz
_lib.kvq_decode_attention.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _f32, _i32,
                                      _P, _sz, _P, _P]
_lib.kvq_decode_attention.restype = ctypes.c_int
_lib.kvq_decode_step.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _f32, _i32, _P,
                                 _sz, _P, _i32, _P]
_lib.kvq_decode_step.restype = ctypes.c_int
_lib.kvq_decode_step_noalloc.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _f32, _i32,
                                         _P, _i32, _P]
_lib.kvq_decode_step_noalloc.restype = ctypes.c_int
_lib.kvq_decode_partials.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _f32, _i32,
                                     _P, _sz, _P, _P]
_lib.kvq_decode_partials.restype = ctypes.c_int
_lib.kvq_decode_merge.argtypes = [_i32, _i32, _i32, _P, _sz, _P, _P]
_lib.kvq_decode_merge.restype = ctypes.c_int
_lib.kvq_decode_attention_ragged.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _P, _P,
                                             _f32, _i32, _P, _sz, _P, _P]
_lib.kvq_decode_attention_ragged.restype = ctypes.c_int
_lib.kvq_decode_partials_ragged.argtypes = [_P, _P, _i32, _i32, _i32, _P, _i64, _P, _P, _P, _P,
                                            _f32, _i32, _P, _sz, _P, _P]
_lib.kvq_decode_partials_ragged.restype = ctypes.c_int
_lib.kvq_dequantize.argtypes = [_P, _P, _i32, _i32, _i64, _i64, _P, _P, _P]
_lib.kvq_stream_read.argtypes = [_P, _sz, _P, _i32, _i32, _i32, _P]
_lib.kvq_mx_quantize_pack.argtypes = [_P, _i32, _i32, _P, _P, _i64, _i64, _i64, _P]
_lib.kvq_mx_quantize_pack.restype = ctypes.c_int
_lib.kvq_mx_dequantize.argtypes = [_P, _i32, _i32, _i64, _i64, _P, _P, _P]
_lib.kvq_mx_dequantize.restype = ctypes.c_int
_lib.kvq_mx_decode_plan.argtypes = [_i32, _i32, _i32, _i64, _i32, _P, _P]
_lib.kvq_mx_decode_plan.restype = ctypes.c_int
_lib.kvq_mx_decode_attention.argtypes = [_P, _i32, _i32, _i32, _P, _i64, _P, _P, _f32, _i32, _P,
                                         _sz, _P, _P]
_lib.kvq_mx_decode_attention.restype = ctypes.c_int
_lib.kvq_stream_read.restype = ctypes.c_int
_lib.kvq_dequantize.restype = ctypes.c_int


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvq_status_string(status)}")


def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


# ----------------------------------------------------------------- containers

@dataclass
class QCfg:
    bits: int = 2
    group: int = 128
    head_dim: int = 128
    n_boost: int = 0
    v_bits: int = 0        # value code width (0: the key width)
    boost_score: int = 0   # Kitty channel importance: 0 range, 1 mean |x|

    @property
    def vb(self) -> int:
        return self.v_bits or self.bits

    def c(self) -> kvq_qcfg:
        return kvq_qcfg(self.bits, self.group, self.head_dim, self.n_boost, self.v_bits,
                        self.boost_score)


@dataclass
class Cache:
    """Packed cache tensors (layout in include/kvq.h).  ``heads`` = B*H_kv.
    With ``page_table`` (int32 ``[heads][pt_stride]``) the tensors are a pool
    of ``t_cap / G`` one-group pages (``Cache.pool``)."""
    cfg: QCfg
    t_cap: int
    heads: int
    k_codes: torch.Tensor
    k_scale: torch.Tensor
    k_min: torch.Tensor
    k_hi: torch.Tensor | None
    k_bidx: torch.Tensor | None
    v_codes: torch.Tensor
    v_scale: torch.Tensor
    v_min: torch.Tensor
    page_table: torch.Tensor | None = None

    FIELDS = ("k_codes", "k_scale", "k_min", "k_hi", "k_bidx", "v_codes", "v_scale", "v_min")

    @staticmethod
    def empty(cfg: QCfg, heads: int, t_cap: int, device="cuda") -> "Cache":
        fpi, v_fpi = 32 // cfg.bits, 32 // cfg.vb
        D, G, T, H = cfg.head_dim, cfg.group, t_cap, heads
        z = dict(device=device)
        return Cache(
            cfg, t_cap, heads,
            k_codes=torch.zeros((H, T, D // fpi), dtype=torch.int32, **z),
            k_scale=torch.zeros((H, T // G, D), dtype=torch.int16, **z),
            k_min=torch.zeros((H, T // G, D), dtype=torch.int16, **z),
            k_hi=torch.zeros((H, T, cfg.n_boost // 16), dtype=torch.int32, **z)
            if cfg.n_boost else None,
            k_bidx=torch.zeros((H, T // G, D), dtype=torch.uint8, **z) if cfg.n_boost else None,
            v_codes=torch.zeros((H, T // v_fpi, D), dtype=torch.int32, **z),
            v_scale=torch.zeros((H, T, D // G), dtype=torch.int16, **z),
            v_min=torch.zeros((H, T, D // G), dtype=torch.int16, **z),
        )

    @staticmethod
    def pool(cfg: QCfg, n_pages: int, page_table: torch.Tensor, device="cuda") -> "Cache":
        """A paged cache: ``n_pages`` one-group pages, and the page of group g
        of head h at ``page_table[h][g]`` (int32 ``[heads][max_groups]``)."""
        c = Cache.empty(cfg, 1, n_pages * cfg.group, device=device)
        c.heads = int(page_table.shape[0])
        c.page_table = page_table.to(torch.int32).contiguous()
        return c

    def heads_view(self, h0: int, n: int) -> "Cache":
        """The cache restricted to heads [h0, h0+n) (same storage)."""
        if self.page_table is not None:
            return Cache(self.cfg, self.t_cap, n,
                         **{f: getattr(self, f) for f in self.FIELDS},
                         page_table=self.page_table[h0:h0 + n])
        sl = {f: (None if getattr(self, f) is None else getattr(self, f)[h0:h0 + n])
              for f in self.FIELDS}
        return Cache(self.cfg, self.t_cap, n, **sl)

    def nbytes(self) -> int:
        return sum(getattr(self, f).numel() * getattr(self, f).element_size()
                   for f in self.FIELDS if getattr(self, f) is not None)

    def c(self) -> kvq_cache:
        pt = self.page_table
        return kvq_cache(*[_ptr(getattr(self, f)) for f in self.FIELDS], self.t_cap,
                         _ptr(pt), 0 if pt is None else int(pt.stride(0)))


def window(k: torch.Tensor | None, v: torch.Tensor | None, n: int) -> kvq_window | None:
    """fp16 window ``[heads][cap][D]`` with the first ``n`` rows valid."""
    if k is None or n == 0:
        return None
    return kvq_window(_ptr(k), _ptr(v), int(n), int(k.shape[1]))


# ----------------------------------------------------------------- entry points

def kvq_quantize_pack(cfg: QCfg, cache: Cache, B: int, H_kv: int, k_src: torch.Tensor,
                      v_src: torch.Tensor, first_group: int, n_groups: int,
                      src_head_stride: int | None = None, stream=None) -> None:
    """fp16 sources ``[B*H_kv][>= n_groups*G][D]`` -> groups [first, first+n)."""
    if src_head_stride is None:
        src_head_stride = k_src.stride(0)
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_quantize_pack(ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_kv,
                                  _ptr(k_src), _ptr(v_src), src_head_stride, first_group,
                                  n_groups, _stream(stream)), "kvq_quantize_pack")


def kvq_decode_plan(cfg: QCfg, B: int, H_q: int, H_kv: int, n_quant_tokens: int,
                    n_chunks: int = 0):
    """(chunks per head, workspace bytes)."""
    nc, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    c_cfg = cfg.c()
    _check(_lib.kvq_decode_plan(ctypes.byref(c_cfg), B, H_q, H_kv, n_quant_tokens, n_chunks,
                                ctypes.byref(nc), ctypes.byref(ws)), "kvq_decode_plan")
    return nc.value, ws.value


def decode_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A decode workspace of ``nbytes`` (from ``kvq_decode_plan``), allocated
    zeroed as the counter bytes at its start require."""
    return torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device=device)


def workspace_status(workspace: torch.Tensor):
    """(stalled blocks, parts poisoned by a bad page) counted in a workspace's
    status words since it was zeroed (synchronizes with the device)."""
    w = workspace.view(torch.int32)[KVQ_WS_STATUS // 4: KVQ_WS_STATUS // 4 + 2].cpu()
    return int(w[0]), int(w[1])


def clear_workspace_status(workspace: torch.Tensor) -> None:
    """Zero the status words of a workspace (asynchronous, on the current stream)."""
    workspace.view(torch.int32)[KVQ_WS_STATUS // 4: KVQ_WS_STATUS // 4 + 2].zero_()


def workspace_records(workspace: torch.Tensor, rows: int, n_parts: int, D: int = 128):
    """The partial records ``[rows][n_parts][D+2]`` (m, l, acc) that follow the
    counter bytes of a workspace (a view)."""
    off = KVQ_WS_COUNTER_BYTES // 4
    return workspace[off: off + rows * n_parts * (D + 2)].view(rows, n_parts, D + 2)


def kvq_decode_workspace_bytes(cfg: QCfg, B: int, H_q: int, H_kv: int, n_quant_tokens: int,
                               n_chunks: int = 0) -> int:
    c_cfg = cfg.c()
    return int(_lib.kvq_decode_workspace_bytes(ctypes.byref(c_cfg), B, H_q, H_kv,
                                               n_quant_tokens, n_chunks))


def kvq_decode_attention(cfg: QCfg, cache: Cache, B: int, H_q: int, H_kv: int,
                         q: torch.Tensor, n_quant_tokens: int, sink: kvq_window | None,
                         res: kvq_window | None, out: torch.Tensor, workspace: torch.Tensor,
                         sm_scale: float = 0.0, n_chunks: int = 0, stream=None) -> None:
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_decode_attention(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, float(sm_scale), int(n_chunks),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _stream(stream)), "kvq_decode_attention")


def kvq_decode_step(cfg: QCfg, cache: Cache, B: int, H_q: int, H_kv: int, q: torch.Tensor,
                    n_quant_tokens: int, sink: kvq_window | None, res: kvq_window | None,
                    out: torch.Tensor, workspace: torch.Tensor, append: bool,
                    sm_scale: float = 0.0, n_chunks: int = 0, stream=None) -> None:
    """Decode step + (when ``append``) the residual group quantized into group
    ``n_quant_tokens / G`` in the same launch where the path supports it."""
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_decode_step(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, float(sm_scale), int(n_chunks),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        1 if append else 0, _stream(stream)), "kvq_decode_step")


def kvq_decode_step_noalloc(cfg: QCfg, cache: Cache, B: int, H_q: int, H_kv: int,
                            q: torch.Tensor, n_quant_tokens: int, sink: kvq_window | None,
                            res: kvq_window | None, out: torch.Tensor, append: bool,
                            sm_scale: float = 0.0, n_chunks: int = 0, stream=None) -> None:
    """kvq_decode_step on the library's own per-GPU scratch array (no
    workspace argument; the call allocates nothing)."""
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_decode_step_noalloc(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, float(sm_scale), int(n_chunks),
        _ptr(out), int(bool(append)), _stream(stream)), "kvq_decode_step_noalloc")


def kvq_decode_partials(cfg: QCfg, cache: Cache, B: int, H_q: int, H_kv: int,
                        q: torch.Tensor, n_quant_tokens: int, sink: kvq_window | None,
                        res: kvq_window | None, workspace: torch.Tensor, sm_scale: float = 0.0,
                        n_chunks: int = 0, stream=None) -> int:
    """Split-K phase only; returns the number of parts per (batch, query head)."""
    c_cfg, c_cache = cfg.c(), cache.c()
    n_parts = ctypes.c_int32(0)
    _check(_lib.kvq_decode_partials(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, float(sm_scale), int(n_chunks),
        _ptr(workspace), workspace.numel() * workspace.element_size(), ctypes.byref(n_parts),
        _stream(stream)), "kvq_decode_partials")
    return n_parts.value


def kvq_decode_attention_ragged(cfg: QCfg, cache: Cache, B: int, H_q: int, H_kv: int,
                                q: torch.Tensor, n_quant_tokens: int,
                                sink: kvq_window | None, res: kvq_window | None,
                                seq_quant: torch.Tensor | None, seq_res: torch.Tensor | None,
                                out: torch.Tensor, workspace: torch.Tensor,
                                sm_scale: float = 0.0, n_chunks: int = 0, stream=None) -> None:
    """Decode with per-sequence lengths (device int32 ``[B]`` tensors or None);
    ``n_quant_tokens`` is the batch's maximum."""
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_decode_attention_ragged(
        ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, _ptr(seq_quant), _ptr(seq_res),
        float(sm_scale), int(n_chunks), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)),
        "kvq_decode_attention_ragged")


def kvq_decode_merge(B: int, H_q: int, n_parts: int, workspace: torch.Tensor,
                     out: torch.Tensor, stream=None) -> None:
    _check(_lib.kvq_decode_merge(B, H_q, n_parts, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _ptr(out),
                                 _stream(stream)), "kvq_decode_merge")


def kvq_dequantize(cfg: QCfg, cache: Cache, B: int, H_kv: int, first_group: int,
                   n_groups: int, k_out: torch.Tensor, v_out: torch.Tensor,
                   stream=None) -> None:
    c_cfg, c_cache = cfg.c(), cache.c()
    _check(_lib.kvq_dequantize(ctypes.byref(c_cfg), ctypes.byref(c_cache), B, H_kv,
                               first_group, n_groups, _ptr(k_out), _ptr(v_out),
                               _stream(stream)), "kvq_dequantize")


@dataclass
class MxCache:
    """MXFP4 cache tensors (layout in include/kvq.h), ``heads`` = B*H_kv."""
    t_cap: int
    heads: int
    k_codes: torch.Tensor
    k_scale: torch.Tensor
    v_codes: torch.Tensor
    v_scale: torch.Tensor

    @staticmethod
    def empty(heads: int, t_cap: int, head_dim: int = 128, device="cuda") -> "MxCache":
        H, T, D = heads, t_cap, head_dim
        z = dict(device=device)
        return MxCache(t_cap, heads,
                       k_codes=torch.zeros((H, T, D // 8), dtype=torch.int32, **z),
                       k_scale=torch.zeros((H, T, D // 32), dtype=torch.uint8, **z),
                       v_codes=torch.zeros((H, T // 8, D), dtype=torch.int32, **z),
                       v_scale=torch.zeros((H, T // 32, D), dtype=torch.uint8, **z))

    def c(self) -> kvq_mx_cache:
        return kvq_mx_cache(_ptr(self.k_codes), _ptr(self.k_scale), _ptr(self.v_codes),
                            _ptr(self.v_scale), self.t_cap)


def kvq_mx_quantize_pack(cache: MxCache, B: int, H_kv: int, k_src: torch.Tensor,
                         v_src: torch.Tensor, first_token: int, n_tokens: int,
                         stream=None) -> None:
    """k_src / v_src: fp16 ``[B*H_kv][>= n_tokens][D]``."""
    c = cache.c()
    _check(_lib.kvq_mx_quantize_pack(ctypes.byref(c), B, H_kv, _ptr(k_src), _ptr(v_src),
                                     k_src.stride(0), first_token, n_tokens, _stream(stream)),
           "kvq_mx_quantize_pack")


def kvq_mx_dequantize(cache: MxCache, B: int, H_kv: int, first_token: int, n_tokens: int,
                      k_out: torch.Tensor, v_out: torch.Tensor, stream=None) -> None:
    c = cache.c()
    _check(_lib.kvq_mx_dequantize(ctypes.byref(c), B, H_kv, first_token, n_tokens, _ptr(k_out),
                                  _ptr(v_out), _stream(stream)), "kvq_mx_dequantize")


def kvq_mx_decode_plan(B: int, H_q: int, H_kv: int, n_quant_tokens: int,
                       n_chunks: int = 0) -> tuple[int, int]:
    """(chunks per head, workspace bytes) of an MXFP4 decode."""
    nc, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    _check(_lib.kvq_mx_decode_plan(B, H_q, H_kv, n_quant_tokens, n_chunks, ctypes.byref(nc),
                                   ctypes.byref(ws)), "kvq_mx_decode_plan")
    return nc.value, ws.value


def kvq_mx_decode_attention(cache: MxCache, B: int, H_q: int, H_kv: int, q: torch.Tensor,
                            n_quant_tokens: int, sink, res, out: torch.Tensor,
                            workspace: torch.Tensor, sm_scale: float = 0.0, n_chunks: int = 0,
                            stream=None) -> None:
    c = cache.c()
    _check(_lib.kvq_mx_decode_attention(
        ctypes.byref(c), B, H_q, H_kv, _ptr(q), n_quant_tokens,
        ctypes.byref(sink) if sink is not None else None,
        ctypes.byref(res) if res is not None else None, ctypes.c_float(sm_scale), n_chunks,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _stream(stream)), "kvq_mx_decode_attention")


def kvq_stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int, threads: int,
                    mode: int = 0, stream=None) -> None:
    """Read every byte of ``src`` once (a measurement aid: the bandwidth a
    plain read reaches); ``sink`` holds at least blocks*threads int32."""
    if sink.numel() < blocks * threads:
        raise ValueError("sink smaller than blocks*threads words")
    _check(_lib.kvq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                blocks, threads, mode, _stream(stream)), "kvq_stream_read")


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments (status returned, not
    raised).  For tests of the argument checks."""
    return getattr(_lib, name)(*args)
