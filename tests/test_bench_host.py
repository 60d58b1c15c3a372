"""Host-side pieces of the benchmark (no GPU): the FLOP count it divides by,
the one-GPU refusal, and the CPU-oracle baseline record."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def visible_pairs(S, Sk, left, right):
    """Brute force: query i sees key j when -left <= j - (i + Sk - S) <= right."""
    i = np.arange(S)[:, None]
    j = np.arange(Sk)[None, :]
    rel = j - (i + Sk - S)
    ok = np.ones((S, Sk), dtype=bool)
    if left is not None:
        ok &= rel >= -left
    if right is not None:
        ok &= rel <= right
    return int(ok.sum())


def test_full_and_causal_nominal_counts():
    B, H, S, D = 2, 3, 64, 16
    assert bench.flops(B, H, S, D, False) == 10.0 * B * H * S * S * D
    assert bench.flops(B, H, S, D, True) == 5.0 * B * H * S * S * D
    # queries and keys of different lengths: S * Sk pairs, minus S^2 / 2 under the causal mask
    assert bench.flops(1, 1, 32, D, False, Sk=96) == 10.0 * 32 * 96 * D
    assert bench.flops(1, 1, 32, D, True, Sk=96) == 10.0 * (32 * 96 - 32 * 32 / 2) * D


@pytest.mark.parametrize("S,Sk,left,right,causal", [
    (40, 40, 7, None, True), (40, 40, 7, 3, False), (24, 56, 10, None, True), (56, 24, 5, 5, False),
    (33, 33, 0, None, True), (17, 50, None, 4, False),
])
def test_window_counts_are_exact(S, Sk, left, right, causal):
    D = 8
    got = bench.flops(1, 1, S, D, causal, Sk=Sk, window=(left, right))
    want = 10.0 * D * visible_pairs(S, Sk, left, 0 if causal else right)
    assert got == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])


def test_cpu_baseline_record():
    from scheduling_persistent_fa_amd.inputs import WORKLOADS
    rec = bench.cpu_baseline(dict(WORKLOADS["full_b1_h1_s256_d64"]), min_seconds=0.0, max_heads=1)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0 and rec["cores"] >= 1
