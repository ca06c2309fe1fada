"""CPU oracle for the low-bit KV cache path -- TEST INFRASTRUCTURE ONLY.

ctypes bindings to ``liboracle_kvq.so`` built from ``kvq_oracle.cpp`` (plain
C++, no GPU code, no code shared with the HIP library).  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package.

Every function works on numpy arrays on the host.  fp16 data travels as raw
``uint16`` bit patterns, packed words as ``uint32``.

Cache layout (per head = b*H_kv + h_kv, ``t_cap`` token slots), the same as
the GPU library's but defined here independently:

* ``k_words``  ``[heads][t_cap][D/fpi]``  key codes packed along channels
* ``k_scale``, ``k_min``  ``[heads][t_cap/G][D]`` fp16 per (group, channel)
* ``k_hi``     ``[heads][t_cap][n_boost/16]`` high two bits of boosted channels
* ``k_bidx``   ``[heads][t_cap/G][D]`` uint8 boosted row or ``n_boost``
* ``v_words``  ``[heads][t_cap/fpi][D]``  value codes packed along tokens
* ``v_scale``, ``v_min``  ``[heads][t_cap][D/G]`` fp16 per (token, channel group)
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle_kvq.so")
# another build of the same source (the sanitizer test's ASan/UBSan build)
_LOAD_PATH = os.environ.get("KVQ_ORACLE_LIB") or _LIB_PATH
_lib = None

BUILD_CMD = [
    "g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
    "-Wall", "-o", _LIB_PATH, _SRC, "-lpthread",
]


def build() -> str:
    """Compile the oracle library in place and return its path."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LOAD_PATH)
    P = ctypes.c_void_p
    i32, i64, u16, f32, f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint16,
                               ctypes.c_float, ctypes.c_double)
    lib.oracle_f16_to_f64.argtypes = [u16]
    lib.oracle_f16_to_f64.restype = f64
    lib.oracle_f16_to_f32.argtypes = [u16]
    lib.oracle_f16_to_f32.restype = f32
    lib.oracle_f32_to_f16.argtypes = [f32]
    lib.oracle_f32_to_f16.restype = u16
    lib.oracle_group_minmax.argtypes = [P, i64, i64, P, P]
    lib.oracle_group_range.argtypes = [u16, u16]
    lib.oracle_group_range.restype = f32
    lib.oracle_group_scale.argtypes = [u16, u16, i32]
    lib.oracle_group_scale.restype = u16
    lib.oracle_code.argtypes = [u16, u16, u16, i32]
    lib.oracle_code.restype = ctypes.c_uint8
    lib.oracle_dequant.argtypes = [i32, u16, u16]
    lib.oracle_dequant.restype = f32
    lib.oracle_quantize_group.argtypes = [P, i64, i64, i32, P, P, P]
    lib.oracle_pack.argtypes = [P, i64, i32, P]
    lib.oracle_unpack.argtypes = [P, i64, i32, P]
    lib.oracle_quantize_pack.argtypes = [i32, i32, i32, i32, i32, i32, i64] + [P] * 8 + [
        i64, P, P, i64, i64, i64, i32]
    lib.oracle_quantize_pack.restype = i32
    lib.oracle_dequantize.argtypes = [i32, i32, i32, i32, i32, i32, i64] + [P] * 8 + [
        i64, i64, i64, P, P, i32]
    lib.oracle_dequantize.restype = i32
    lib.oracle_attention_fp64.argtypes = [P, P, P, i64, i32, f64, P]
    lib.oracle_attention_split_merge.argtypes = [P, P, P, i64, i32, f64, i64, P]
    lib.oracle_decode_attention.argtypes = [i32, i32, i32, i32, i32, i32, i64] + [P] * 8 + [
        i32, i32, i32, P, i64, P, P, i32, i32, P, P, i32, i32, f64, P, i32]
    lib.oracle_decode_attention.restype = i32
    u8 = ctypes.c_uint8
    lib.oracle_fp4_value.argtypes = [u8]
    lib.oracle_fp4_value.restype = f64
    lib.oracle_fp4_encode.argtypes = [f64]
    lib.oracle_fp4_encode.restype = u8
    lib.oracle_mx_exponent.argtypes = [P, i64, i64]
    lib.oracle_mx_exponent.restype = i32
    lib.oracle_mx_dequant.argtypes = [u8, u8]
    lib.oracle_mx_dequant.restype = f32
    lib.oracle_mx_quantize_pack.argtypes = [i32, i64, P, P, P, P, i64, P, P, i64, i64, i64, i32]
    lib.oracle_mx_quantize_pack.restype = i32
    lib.oracle_mx_dequantize.argtypes = [i32, i64, P, P, P, P, i64, i64, i64, P, P, i32]
    lib.oracle_mx_dequantize.restype = i32
    lib.oracle_mx_decode_attention.argtypes = [i32, i64, P, P, P, P, i32, i32, i32, P, i64, P,
                                               P, i32, i32, P, P, i32, i32, f64, P, i32]
    lib.oracle_mx_decode_attention.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalar / small helpers (used by the pin tests)
# --------------------------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def f32_to_f16(x: float) -> int:
    return int(_load().oracle_f32_to_f16(float(np.float32(x))))


def group_minmax(x_bits: np.ndarray):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    mn, mx = np.zeros(1, np.uint16), np.zeros(1, np.uint16)
    _load().oracle_group_minmax(_ptr(x), x.size, 1, _ptr(mn), _ptr(mx))
    return int(mn[0]), int(mx[0])


def group_range(mn_bits: int, mx_bits: int) -> float:
    return float(_load().oracle_group_range(mn_bits, mx_bits))


def quantize_group(x_bits: np.ndarray, bits: int):
    """(min fp16 bits, scale fp16 bits, codes uint8) of one group."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    mn, s = np.zeros(1, np.uint16), np.zeros(1, np.uint16)
    codes = np.zeros(x.size, np.uint8)
    _load().oracle_quantize_group(_ptr(x), x.size, 1, bits, _ptr(mn), _ptr(s), _ptr(codes))
    return int(mn[0]), int(s[0]), codes


def dequant(q: int, s_bits: int, mn_bits: int) -> float:
    return float(_load().oracle_dequant(int(q), int(s_bits), int(mn_bits)))


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(c.size * bits // 32, np.uint32)
    _load().oracle_pack(_ptr(c), c.size, bits, _ptr(out))
    return out


def unpack(words: np.ndarray, n_codes: int, bits: int) -> np.ndarray:
    w = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.zeros(n_codes, np.uint8)
    _load().oracle_unpack(_ptr(w), n_codes, bits, _ptr(out))
    return out


def attention_fp64(q, K, V, sm: float) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    out = np.zeros(q.shape[-1], np.float64)
    _load().oracle_attention_fp64(_ptr(q), _ptr(K), _ptr(V), K.shape[0], q.shape[-1], sm, _ptr(out))
    return out


def attention_split_merge(q, K, V, sm: float, chunk: int) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    out = np.zeros(q.shape[-1], np.float64)
    _load().oracle_attention_split_merge(_ptr(q), _ptr(K), _ptr(V), K.shape[0], q.shape[-1],
                                         sm, chunk, _ptr(out))
    return out


# --------------------------------------------------------------------------
# whole cache
# --------------------------------------------------------------------------

@dataclass
class Cache:
    bits: int
    group: int
    head_dim: int
    n_boost: int
    t_cap: int
    n_heads: int
    k_words: np.ndarray
    k_scale: np.ndarray
    k_min: np.ndarray
    k_hi: np.ndarray | None
    k_bidx: np.ndarray | None
    v_words: np.ndarray
    v_scale: np.ndarray
    v_min: np.ndarray
    v_bits: int = 0       # value code width (0: the key width)
    score: int = 0        # Kitty channel importance: 0 range, 1 mean |x|

    @property
    def vb(self) -> int:
        return self.v_bits or self.bits

    @property
    def fpi(self) -> int:
        """Key codes per word."""
        return 32 // self.bits

    @property
    def v_fpi(self) -> int:
        """Value codes per word."""
        return 32 // self.vb

    def _args(self):
        return [self.bits, self.vb, self.group, self.head_dim, self.n_boost, self.score,
                self.t_cap,
                _ptr(self.k_words), _ptr(self.k_scale), _ptr(self.k_min), _ptr(self.k_hi),
                _ptr(self.k_bidx), _ptr(self.v_words), _ptr(self.v_scale), _ptr(self.v_min)]


def empty_cache(bits: int, group: int, head_dim: int, n_boost: int, t_cap: int,
                n_heads: int, v_bits: int = 0, score: int = 0) -> Cache:
    """Key codes of ``bits`` bits, value codes of ``v_bits`` (0: the same)."""
    fpi, v_fpi = 32 // bits, 32 // (v_bits or bits)
    H, T, D, G = n_heads, t_cap, head_dim, group
    return Cache(
        bits, group, head_dim, n_boost, t_cap, n_heads,
        k_words=np.zeros((H, T, D // fpi), np.uint32),
        k_scale=np.zeros((H, T // G, D), np.uint16),
        k_min=np.zeros((H, T // G, D), np.uint16),
        k_hi=np.zeros((H, T, n_boost // 16), np.uint32) if n_boost else None,
        k_bidx=np.zeros((H, T // G, D), np.uint8) if n_boost else None,
        v_words=np.zeros((H, T // v_fpi, D), np.uint32),
        v_scale=np.zeros((H, T, D // G), np.uint16),
        v_min=np.zeros((H, T, D // G), np.uint16),
        v_bits=v_bits, score=score,
    )


def quantize_pack(cache: Cache, k_src: np.ndarray, v_src: np.ndarray, first_group: int,
                  n_groups: int, n_threads: int = 0) -> None:
    """Quantize groups [first_group, first_group+n_groups) of every head.

    k_src, v_src: fp16 bits ``[heads][>= n_groups*G][D]``.
    """
    k = np.ascontiguousarray(k_src, np.uint16)
    v = np.ascontiguousarray(v_src, np.uint16)
    assert k.shape == v.shape and k.shape[0] == cache.n_heads
    rc = _load().oracle_quantize_pack(*cache._args(), cache.n_heads, _ptr(k), _ptr(v),
                                      k.shape[1] * k.shape[2], first_group, n_groups, n_threads)
    if rc:
        raise ValueError("oracle_quantize_pack: bad configuration")


def dequantize(cache: Cache, first_group: int, n_groups: int, n_threads: int = 0):
    n = n_groups * cache.group
    k = np.zeros((cache.n_heads, n, cache.head_dim), np.float32)
    v = np.zeros_like(k)
    rc = _load().oracle_dequantize(*cache._args(), cache.n_heads, first_group, n_groups,
                                   _ptr(k), _ptr(v), n_threads)
    if rc:
        raise ValueError("oracle_dequantize: bad configuration")
    return k, v


def decode_attention(cache: Cache, B: int, H_q: int, H_kv: int, q: np.ndarray, n_quant: int,
                     k_sink=None, v_sink=None, n_sink: int = 0, k_res=None, v_res=None,
                     n_res: int = 0, sm: float = 0.0, n_threads: int = 0) -> np.ndarray:
    """fp64 attention output ``[B][H_q][D]``; windows are fp16 bits ``[heads][cap][D]``."""
    D = cache.head_dim
    q = np.ascontiguousarray(q, np.uint16)
    ks = None if k_sink is None else np.ascontiguousarray(k_sink, np.uint16)
    vs = None if v_sink is None else np.ascontiguousarray(v_sink, np.uint16)
    kr = None if k_res is None else np.ascontiguousarray(k_res, np.uint16)
    vr = None if v_res is None else np.ascontiguousarray(v_res, np.uint16)
    sink_cap = 0 if ks is None else ks.shape[1]
    res_cap = 0 if kr is None else kr.shape[1]
    out = np.zeros((B, H_q, D), np.float64)
    rc = _load().oracle_decode_attention(*cache._args(), B, H_q, H_kv, _ptr(q), n_quant,
                                         _ptr(ks), _ptr(vs), n_sink, sink_cap, _ptr(kr),
                                         _ptr(vr), n_res, res_cap, sm, _ptr(out), n_threads)
    if rc:
        raise ValueError("oracle_decode_attention: bad configuration")
    return out


# --------------------------------------------------------------------------
# MXFP4 cache (32-value blocks, E8M0 scale, E2M1 values); layout per head:
#   k_words [t_cap][D/8] u32, k_scale [t_cap][D/32] u8 (blocks of 32 channels)
#   v_words [t_cap/8][D] u32, v_scale [t_cap/32][D] u8 (blocks of 32 tokens)
# --------------------------------------------------------------------------

def fp4_value(code: int) -> float:
    return float(_load().oracle_fp4_value(int(code)))


def fp4_encode(v: float) -> int:
    return int(_load().oracle_fp4_encode(float(v)))


def mx_exponent(x_bits: np.ndarray) -> int:
    """Shared exponent E of a block of fp16 values (bits)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    return int(_load().oracle_mx_exponent(_ptr(x), x.size, 1))


def mx_dequant(code: int, e8m0: int) -> float:
    return float(_load().oracle_mx_dequant(int(code), int(e8m0)))


@dataclass
class MxCache:
    head_dim: int
    t_cap: int
    n_heads: int
    k_words: np.ndarray
    k_scale: np.ndarray
    v_words: np.ndarray
    v_scale: np.ndarray

    def _args(self):
        return [self.head_dim, self.t_cap, _ptr(self.k_words), _ptr(self.k_scale),
                _ptr(self.v_words), _ptr(self.v_scale)]


def mx_empty_cache(head_dim: int, t_cap: int, n_heads: int) -> MxCache:
    H, T, D = n_heads, t_cap, head_dim
    return MxCache(D, T, H, k_words=np.zeros((H, T, D // 8), np.uint32),
                   k_scale=np.zeros((H, T, D // 32), np.uint8),
                   v_words=np.zeros((H, T // 8, D), np.uint32),
                   v_scale=np.zeros((H, T // 32, D), np.uint8))


def mx_quantize_pack(cache: MxCache, k_src: np.ndarray, v_src: np.ndarray, t0: int, n: int,
                     n_threads: int = 0) -> None:
    """Quantize tokens [t0, t0+n) of every head from fp16 bits [heads][>= n][D]."""
    k = np.ascontiguousarray(k_src, np.uint16)
    v = np.ascontiguousarray(v_src, np.uint16)
    assert k.shape == v.shape and k.shape[0] == cache.n_heads
    rc = _load().oracle_mx_quantize_pack(*cache._args(), cache.n_heads, _ptr(k), _ptr(v),
                                         k.shape[1] * k.shape[2], t0, n, n_threads)
    if rc:
        raise ValueError("oracle_mx_quantize_pack: bad configuration")


def mx_dequantize(cache: MxCache, t0: int, n: int, n_threads: int = 0):
    k = np.zeros((cache.n_heads, n, cache.head_dim), np.float32)
    v = np.zeros_like(k)
    rc = _load().oracle_mx_dequantize(*cache._args(), cache.n_heads, t0, n, _ptr(k), _ptr(v),
                                      n_threads)
    if rc:
        raise ValueError("oracle_mx_dequantize: bad configuration")
    return k, v


def mx_decode_attention(cache: MxCache, B: int, H_q: int, H_kv: int, q: np.ndarray,
                        n_quant: int, k_sink=None, v_sink=None, n_sink: int = 0, k_res=None,
                        v_res=None, n_res: int = 0, sm: float = 0.0,
                        n_threads: int = 0) -> np.ndarray:
    """fp64 attention output ``[B][H_q][D]`` over the MXFP4 cache."""
    D = cache.head_dim
    q = np.ascontiguousarray(q, np.uint16)
    ks = None if k_sink is None else np.ascontiguousarray(k_sink, np.uint16)
    vs = None if v_sink is None else np.ascontiguousarray(v_sink, np.uint16)
    kr = None if k_res is None else np.ascontiguousarray(k_res, np.uint16)
    vr = None if v_res is None else np.ascontiguousarray(v_res, np.uint16)
    out = np.zeros((B, H_q, D), np.float64)
    rc = _load().oracle_mx_decode_attention(
        *cache._args(), B, H_q, H_kv, _ptr(q), n_quant, _ptr(ks), _ptr(vs), n_sink,
        0 if ks is None else ks.shape[1], _ptr(kr), _ptr(vr), n_res,
        0 if kr is None else kr.shape[1], sm, _ptr(out), n_threads)
    if rc:
        raise ValueError("oracle_mx_decode_attention: bad configuration")
    return out
