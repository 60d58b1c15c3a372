"""Seeded synthetic inputs for the attention backward workloads.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the attention arithmetic, so both the CPU oracle (through the tests)
and the GPU path use it without sharing any computation.

Recipe: numpy ``default_rng(seed)``; fp32 standard normals drawn in the order
Q, K, V, dO, multiplied by ``std``; then rounded to bfloat16 with
round-to-nearest-even.  Q and dO have shape [B, Hq, S, D]; K and V have shape
[B, Hkv, Sk, D] (Sk = S unless given); all contiguous row-major (BHSD).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class AttnInputs:
    """bfloat16 bit patterns (uint16) of Q, K, V, dO plus the problem sizes."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    Sk: int = 0

    def as_f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


def make_inputs(B: int, Hq: int, Hkv: int, S: int, D: int, seed: int = 0, std: float = 1.0,
                Sk: int | None = None) -> AttnInputs:
    Sk = S if Sk is None else Sk
    rng = np.random.default_rng(seed)
    shapes = {"q": (B, Hq, S, D), "k": (B, Hkv, Sk, D), "v": (B, Hkv, Sk, D), "do": (B, Hq, S, D)}
    out = {}
    for name in ("q", "k", "v", "do"):
        x = rng.standard_normal(size=shapes[name], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[name] = f32_to_bf16_bits(x)
    return AttnInputs(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, Sk=Sk, **out)


# Benchmark workloads, named by mask and sizes: (B, Hq, Hkv, S, D, causal, tile, std).
WORKLOADS = {
    "full_b1_h1_s256_d64": dict(B=1, Hq=1, Hkv=1, S=256, D=64, causal=False, tile=64, std=1.0),
    "causal_b4_h16_s2048_d128": dict(B=4, Hq=16, Hkv=16, S=2048, D=128, causal=True, tile=128, std=1.0),
    "full_b2_h24_s4096_d64": dict(B=2, Hq=24, Hkv=24, S=4096, D=64, causal=False, tile=128, std=1.0),
    "full_b1_h16_s16384_d128": dict(B=1, Hq=16, Hkv=16, S=16384, D=128, causal=False, tile=128, std=1.0),
    "causal_b1_h16_s16384_d128": dict(B=1, Hq=16, Hkv=16, S=16384, D=128, causal=True, tile=128, std=1.0),
    "gqa_causal_b1_hq32_hkv8_s8192_d128": dict(B=1, Hq=32, Hkv=8, S=8192, D=128, causal=True, tile=128, std=0.5),
    # queries and keys of different lengths (S query rows, Sk key rows): cross
    # attention, and a causal continuation aligned at the bottom right
    "cross_b1_h16_q4096_k16384_d128": dict(B=1, Hq=16, Hkv=16, S=4096, Sk=16384, D=128, causal=False, tile=128, std=1.0),
    "causal_b1_h16_q4096_k16384_d128": dict(B=1, Hq=16, Hkv=16, S=4096, Sk=16384, D=128, causal=True, tile=128,
                                            std=1.0),
    # sliding-window causal attention: each query sees its own key and the
    # 4095 before it (a 4096-key window)
    "sliding_b1_h16_s16384_w4096_d128": dict(B=1, Hq=16, Hkv=16, S=16384, D=128, causal=True, window=(4095, 0),
                                             tile=128, std=1.0),
}
