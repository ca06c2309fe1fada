"""Seeded synthetic inputs for the low-bit KV cache path.

Test and benchmark infrastructure shared by the GPU-path tests and the oracle
tests.  It holds workload shapes and random-number recipes only -- none of the
quantization or attention arithmetic.

Distributions stand in for the Llama-class decode workloads of the KIVI,
Kitty and BitDecoding pages (no model or dataset is used): Q ~ N(0,1),
V ~ N(0,1), K ~ N(0,1) with a few fixed outlier channels per kv head whose
values are scaled by a large factor for every token (the "some fixed channels
have very large magnitudes" observation of the KIVI page, Step 1, and the
Kitty page, section 3.2).  Every tensor is drawn in fp32 by torch's seeded
generator on the requested device and rounded to fp16 (round to nearest
even).  A tensor is addressed by (workload seed, kv head, kind), so one head
can be regenerated without the others.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    D: int
    T: int            # quantized tokens per head
    R: int            # fp16 residual (local) tokens per head
    S: int            # fp16 sink tokens per head
    bits: int
    G: int
    n_boost: int      # key channels kept at 4 bits per group (0 = plain KIVI)
    outlier: str      # outlier-channel recipe, see outlier_channels()
    seed: int
    min_chunks: int = 0   # smallest split-K chunk count per head the workload asks for
    note: str = ""
    v_bits: int = 0       # value code width (0: the key width)
    boost_score: int = 0  # Kitty channel importance: 0 range, 1 mean |x|

    @property
    def heads(self) -> int:
        return self.B * self.H_kv

    @property
    def gqa(self) -> int:
        return self.H_q // self.H_kv


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_t512_g32_2bit", B=1, H_q=1, H_kv=1, D=128, T=512, R=32, S=0, bits=2,
                 G=32, n_boost=0, outlier="fixed4x15", seed=1001,
                 note="quantize all 16 groups + one decode step"),
        Workload("llama3_8b_t32k_2bit", B=8, H_q=32, H_kv=8, D=128, T=32768, R=128, S=0, bits=2,
                 G=128, n_boost=0, outlier="rand5x10_20", seed=1002,
                 note="one decode step + append-group quantize"),
        Workload("llama3_8b_t8k_b32_4bit", B=32, H_q=32, H_kv=8, D=128, T=8192, R=128, S=0,
                 bits=4, G=128, n_boost=0, outlier="rand5x10_20", seed=1003,
                 note="decode step + streaming append of 128-token groups"),
        Workload("kitty_t128k_h64_boost16", B=16, H_q=64, H_kv=8, D=128, T=131072, R=128, S=32,
                 bits=2, G=128, n_boost=16, outlier="fixed8x20", seed=1004,
                 note="16 of 128 key channels 4-bit per group; 32 sink + 128 local fp16"),
        Workload("long_t1m_2bit_splitk", B=1, H_q=32, H_kv=8, D=128, T=1048576, R=128, S=0,
                 bits=2, G=128, n_boost=0, outlier="rand5x10_20", seed=1005, min_chunks=256,
                 note=">= 256 KV chunks per head, fp32 log-sum-exp merge"),
    ]
}

# tensor kinds inside one head's stream
_K_QUANT, _V_QUANT, _K_RES, _V_RES, _K_SINK, _V_SINK = range(6)
_Q = 15


def _seed(base: int, head: int, kind: int) -> int:
    return (base * 1_000_003 + head * 16 + kind) & 0x7FFF_FFFF_FFFF


def outlier_channels(w: Workload, kv_head: int):
    """(channel indices, multipliers) of kv head ``kv_head`` (= b*H_kv + h)."""
    if w.outlier == "fixed4x15":
        return np.array([3, 17, 64, 100]), np.full(4, 15.0)
    if w.outlier == "fixed8x20":
        rng = np.random.default_rng([w.seed, kv_head, 7])
        return np.sort(rng.choice(w.D, 8, replace=False)), np.full(8, 20.0)
    if w.outlier == "rand5x10_20":
        rng = np.random.default_rng([w.seed, kv_head, 7])
        n = int(round(0.04 * w.D))
        return np.sort(rng.choice(w.D, n, replace=False)), rng.uniform(10.0, 20.0, n)
    if w.outlier == "none":
        return np.zeros(0, np.int64), np.zeros(0)
    raise ValueError(w.outlier)


def _normal(n_rows: int, D: int, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n_rows, D), generator=g, device=device, dtype=torch.float32)


def _key_rows(w: Workload, kv_head: int, n_rows: int, kind: int, device) -> torch.Tensor:
    x = _normal(n_rows, w.D, _seed(w.seed, kv_head, kind), device)
    ch, mult = outlier_channels(w, kv_head)
    if len(ch):
        scale = torch.ones(w.D, dtype=torch.float32)
        scale[torch.as_tensor(ch)] = torch.as_tensor(mult, dtype=torch.float32)
        x = x * scale.to(device)
    return x.to(torch.float16)


def _value_rows(w: Workload, kv_head: int, n_rows: int, kind: int, device) -> torch.Tensor:
    return _normal(n_rows, w.D, _seed(w.seed, kv_head, kind), device).to(torch.float16)


def head_kv(w: Workload, kv_head: int, device="cpu", n_tokens: int | None = None):
    """fp16 source K and V ``[n_tokens][D]`` of the quantized region of one head."""
    n = w.T if n_tokens is None else n_tokens
    return (_key_rows(w, kv_head, n, _K_QUANT, device),
            _value_rows(w, kv_head, n, _V_QUANT, device))


def head_windows(w: Workload, kv_head: int, device="cpu"):
    """fp16 (k_sink, v_sink, k_res, v_res) of one head, ``[S or R][D]``."""
    return (_key_rows(w, kv_head, w.S, _K_SINK, device),
            _value_rows(w, kv_head, w.S, _V_SINK, device),
            _key_rows(w, kv_head, w.R, _K_RES, device),
            _value_rows(w, kv_head, w.R, _V_RES, device))


def query(w: Workload, device="cpu") -> torch.Tensor:
    """fp16 query ``[B][H_q][D]``."""
    return _normal(w.B * w.H_q, w.D, _seed(w.seed, 0, _Q), device).to(torch.float16).view(
        w.B, w.H_q, w.D)


def shrink(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity-test shapes)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def as_bits(t: torch.Tensor) -> np.ndarray:
    """fp16 tensor -> host numpy uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
