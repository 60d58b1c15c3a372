"""The float64 oracle over whole tensors at the workload sizes.

Calls ``oracle.attention.backward`` once per (batch, query head), concurrently
on the host cores (one BLAS thread per worker), and assembles full dQ, dK and
dV; dK/dV of a key/value head are the float64 sums of its query heads'
contributions in ascending head order.  Nothing here computes attention
itself: every number comes from the oracle.
"""
from __future__ import annotations

import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import attention as A


def host_workers(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def full_reference(inp, causal: bool, window=None, label: str = "") -> dict:
    """dq [B,Hq,Sq,D], dk and dv [B,Hkv,Sk,D] (float64) for seeded inputs
    ``inp`` (scheduling_persistent_fa_amd.inputs.AttnInputs)."""
    from threadpoolctl import threadpool_limits
    q, k, v, do = (inp.as_f64(n) for n in ("q", "k", "v", "do"))
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros_like(q)
    parts = {}
    done = [0]
    t0 = time.time()

    def one(bh):
        b, hq = bh
        hk = hq // g
        r = A.backward(q[b:b + 1, hq:hq + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1], do[b:b + 1, hq:hq + 1],
                       scale, causal, window=window)
        dq[b, hq] = r["dq"][0, 0]
        parts[(b, hq)] = (r["dk"][0, 0], r["dv"][0, 0])
        done[0] += 1
        if done[0] % max(1, (B * Hq) // 4) == 0:
            print(f"  oracle {label}: {done[0]}/{B * Hq} heads, {time.time() - t0:.0f} s", flush=True)
            sys.stdout.flush()

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=host_workers()) as ex:
            list(ex.map(one, [(b, hq) for b in range(B) for hq in range(Hq)]))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for hq in range(Hq):  # ascending query head within each group
            pk, pv = parts.pop((b, hq))
            dk[b, hq // g] += pk
            dv[b, hq // g] += pv
    return {"dq": dq, "dk": dk, "dv": dv}
