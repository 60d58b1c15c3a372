"""Shared helpers of the GPU tests: seeded inputs on the device and the
tolerance metric max|err| / max|ref|."""
from __future__ import annotations

import math
import sys

import numpy as np

from scheduling_persistent_fa_amd.inputs import bf16_bits_to_f32, make_inputs

TOL = 2e-2  # max|gpu - oracle| / max|oracle| for bf16 inputs with fp32 accumulation


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


class DeviceProblem:
    """Seeded inputs uploaded to the GPU plus their exact float64 values."""

    def __init__(self, B, Hq, Hkv, S, D, causal, std=1.0, seed=0, Sk=None):
        import torch
        from scheduling_persistent_fa_amd.attention import bf16_from_bits
        self.B, self.Hq, self.Hkv, self.S, self.D, self.causal = B, Hq, Hkv, S, D, causal
        self.Sk = S if Sk is None else Sk
        self.scale = 1.0 / math.sqrt(D)
        self.inp = make_inputs(B, Hq, Hkv, S, D, seed=seed, std=std, Sk=Sk)
        self.q = bf16_from_bits(self.inp.q)
        self.k = bf16_from_bits(self.inp.k)
        self.v = bf16_from_bits(self.inp.v)
        self.do = bf16_from_bits(self.inp.do)
        torch.cuda.synchronize()

    def f64(self, name):
        return bf16_bits_to_f32(getattr(self.inp, name)).astype(np.float64)
