#!/usr/bin/env python3
"""Deterministic attention backward on one MI355X: TFLOP/s, % of the dense
bf16 matrix-core peak, and the ratio to the non-deterministic atomic variant.

A step is one full backward pass through the C ABI (Delta preprocess,
persistent backward kernel, dQ finalize) over one batch of seeded synthetic
bf16 inputs already resident in device memory.  FLOPs per step are
10 * B * Hq * S^2 * D, halved for the causal mask.  Every deterministic
schedule and every atomic walk of the workload is timed; the reported value is
the best deterministic schedule.  The persistent kernel is also timed on its
own with HIP events recorded on the launch stream, for the roofline.  By
default the causal mask at the same sizes is timed in the same run and
reported under "also", with its own roofline.  Every timed step writes its
own output buffers, and all of them are compared bit for bit with the
warm-up result ("repeat_bitwise").

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix-core peak (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "deterministic attn-bwd TFLOP/s (1 GPU) + % of bf16 MFMA peak + ratio vs atomic"
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "bwd_kernel_counters.json")


def flops(B, Hq, S, D, causal, Sk=None, window=None):
    """Nominal backward FLOPs: 10 * B * Hq * D per visible (query, key) pair,
    counting S * Sk pairs, minus S^2 / 2 under the causal mask (which for
    Sk = S is the usual halving).  With a window (left, right) the visible
    pairs are counted exactly: query i sees keys max(0, i + off - left) ..
    min(Sk - 1, i + off + right), off = Sk - S."""
    Sk = S if Sk is None else Sk
    if window is None:
        pairs = S * Sk - (S * S / 2 if causal else 0)
    else:
        import numpy as np
        left, right = window
        right = 0 if causal else right
        c = np.arange(S, dtype=np.int64) + (Sk - S)
        lo = np.zeros_like(c) if left is None else np.maximum(0, c - left)
        hi = np.full_like(c, Sk - 1) if right is None else np.minimum(Sk - 1, c + right)
        pairs = float(np.maximum(0, hi - lo + 1).sum())
    return 10.0 * B * Hq * D * pairs


def cpu_baseline(wl, min_seconds=10.0, max_heads=8):
    """The float64 oracle on a bounded sample of the workload: whole (batch, head)
    slices, one after another, until about ``min_seconds`` of CPU work."""
    import numpy as np
    from oracle import attention as A
    from scheduling_persistent_fa_amd.inputs import bf16_bits_to_f32, make_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max([p.get("num_threads", 1) for p in blas_pools] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in blas_pools})) or "none"
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores, blas = int(os.environ.get("OMP_NUM_THREADS", "1")), "unknown"
    S, D, causal = wl["S"], wl["D"], wl["causal"]
    Sk, window = wl.get("Sk", S), wl.get("window")
    f64 = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    heads, dt = 0, 0.0
    while heads < max_heads and (heads == 0 or dt < min_seconds):
        inp = make_inputs(1, 1, 1, S, D, seed=heads, std=wl["std"], Sk=Sk)
        q, k, v, do = (f64(x) for x in (inp.q, inp.k, inp.v, inp.do))
        t0 = time.perf_counter()
        A.backward(q, k, v, do, 1.0 / math.sqrt(D), causal, window=window)
        dt += time.perf_counter() - t0
        heads += 1
    mask = ("causal" if causal else "full") + (f" window={window}" if window else "")
    return {"value": heads * flops(1, 1, S, D, causal, Sk, window) / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads} (batch, head) slices of the workload (S={S} Sk={Sk} D={D} "
                      f"{mask}), float64 forward+backward, {blas} BLAS, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_b1_h16_s16384_d128")
    ap.add_argument("--also", default="causal_b1_h16_s16384_d128",
                    help="comma list of further workloads timed in the same run and reported under 'also' "
                         "(default: the causal mask at the same sizes); empty for none")
    ap.add_argument("--schedules", default="", help="comma list (serial,desc_q,shift,sym_shift); default: all for the mask")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-atomic", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates HBM counters)")
    ap.add_argument("--block", action="store_true",
                    help="instead: fwd+bwd of a synthetic transformer block around the attention op "
                         "(deterministic vs atomic backward); prints its own JSON line")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe << 20, "launches": 3}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 (the work would "
                                   "shard by (batch, kv head), with no exchange between GPUs)"}))
        sys.exit(2)
    if args.block:
        block_bench(args)
        return

    first = bench_workload(args.workload, args)
    line = {
        "metric": METRIC,
        "value": round(first["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(first["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    line.update({k: v for k, v in first.items() if k not in ("value", "ms_per_step", "wl")})
    also = [w for w in args.also.split(",") if w and w != args.workload]
    if also:
        line["also"] = {}
        for name in also:
            r = bench_workload(name, args)
            line["also"][name] = {"value": round(r["value"], 2), "ms_per_step": round(r["ms_per_step"], 4),
                                  **{k: v for k, v in r.items() if k not in ("value", "ms_per_step", "wl")}}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(first["wl"])
    print(json.dumps(line), flush=True)


def bench_workload(workload, args):
    """Times every deterministic schedule and atomic walk of one workload;
    returns the fields of its JSON record (value = best deterministic)."""
    import torch
    from scheduling_persistent_fa_amd import _lib
    from scheduling_persistent_fa_amd.attention import attn_bwd, attn_fwd, bf16_from_bits, device_info, make_opts
    from scheduling_persistent_fa_amd.inputs import WORKLOADS, make_inputs

    wl = dict(WORKLOADS[workload])
    B, Hq, Hkv, S, D, causal, tile = wl["B"], wl["Hq"], wl["Hkv"], wl["S"], wl["D"], wl["causal"], wl["tile"]
    Sk, window = wl.get("Sk", S), wl.get("window")
    torch.cuda.set_device(0)
    info = device_info(0)
    inp = make_inputs(B, Hq, Hkv, S, D, seed=0, std=wl["std"], Sk=Sk)
    q, k, v, do = (bf16_from_bits(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    o, lse = attn_fwd(q, k, v, causal, window=window)
    torch.cuda.synchronize()
    fl = flops(B, Hq, S, D, causal, Sk, window)
    # one output set per timed step, so that every timed step's bits are checked
    outs = [(torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) for _ in range(args.steps)]

    # shift needs a full mask; symmetric shift pairs query tiles p, N-1-p and needs N even
    fast = ["shift"] if not causal else (["sym_shift"] if (S // tile) % 2 == 0 else [])
    if window is not None:
        # a sliding band (left, 0) also takes the band shift schedule
        fast = ["shift"] if window[1] == 0 or causal else []
    det_names = ["serial", "desc_q"] + fast
    if args.schedules:
        det_names = [s for s in args.schedules.split(",") if s]
    ids = {"serial": _lib.SERIAL, "desc_q": _lib.DESC_Q, "shift": _lib.SHIFT, "sym_shift": _lib.SYM_SHIFT}
    runs = [(n, ids[n], -1) for n in det_names]
    if not args.no_atomic:
        walks = ["serial", "desc_q"] + fast
        runs += [(f"atomic[{w}]", _lib.ATOMIC, ids[w]) for w in walks]

    stream = torch.cuda.current_stream()
    results = {}
    for name, sched, walk in runs:
        print(f"[bench] {workload} {name}", file=sys.stderr, flush=True)
        base_opts = dict(tile=tile, atomic_walk=walk)
        dq, dk, dv = outs[0]
        for _ in range(args.warmup):
            attn_bwd(q, k, v, o, do, lse, causal, sched, dq=dq, dk=dk, dv=dv, opts=make_opts(**base_opts),
                     window=window)
        ref_bits = dq.view(torch.int16).clone(), dk.view(torch.int16).clone(), dv.view(torch.int16).clone()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a_, b_ in evs:  # materialise the underlying HIP events
            a_.record(stream)
            b_.record(stream)
        opts = [make_opts(events=e, **base_opts) for e in evs]
        t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_beg.record(stream)
        for i in range(args.steps):
            dq, dk, dv = outs[i]
            calls[i][0].record(stream)
            attn_bwd(q, k, v, o, do, lse, causal, sched, dq=dq, dk=dk, dv=dv, opts=opts[i], window=window)
            calls[i][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms = t_beg.elapsed_time(t_end) / args.steps
        kms_each = [a_.elapsed_time(b_) for a_, b_ in evs]
        step_each = sorted(a_.elapsed_time(b_) for a_, b_ in calls)
        kms = sum(kms_each) / args.steps
        # every timed step's dQ, dK, dV against the last warm-up run's bits
        same = all(torch.equal(x.view(torch.int16), r) for out in outs for x, r in zip(out, ref_bits))
        pct = lambda xs, p: xs[min(len(xs) - 1, max(0, int(round(p * (len(xs) - 1)))))]
        rec = {"ms_per_step": ms, "tflops": fl / (ms * 1e-3) / 1e12, "kernel_ms": kms,
               "kernel_tflops": fl / (kms * 1e-3) / 1e12, "repeat_bitwise": bool(same),
               # per-step call times: the median and the 10th / 90th percentiles as TFLOP/s
               "tflops_p50": fl / (pct(step_each, 0.5) * 1e-3) / 1e12,
               "tflops_p10": fl / (pct(step_each, 0.9) * 1e-3) / 1e12,
               "tflops_p90": fl / (pct(step_each, 0.1) * 1e-3) / 1e12}
        if sched != _lib.ATOMIC:
            dq, dk, dv = outs[0]
            stall = torch.zeros(2 * info["num_cu"], dtype=torch.int64, device="cuda")
            ke = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ke[0].record(stream)  # materialise the underlying HIP events
            ke[1].record(stream)
            attn_bwd(q, k, v, o, do, lse, causal, sched, dq=dq, dk=dk, dv=dv,
                     opts=make_opts(stall=stall, sync_check=True, events=ke, **base_opts), window=window)
            x_ = stall.view(-1, 2).double()
            st = x_.sum(0).tolist()
            rec["sem_stall_frac"] = st[0] / max(st[1], 1.0)
            # shader clock under this load: in-kernel s_memtime cycles over the launch's event time
            rec["sclk_ghz_est"] = x_[:, 1].max().item() / (ke[0].elapsed_time(ke[1]) * 1e6)
        results[name] = rec
        print(f"[bench]   {ms:.3f} ms/step  {rec['tflops']:.1f} TFLOP/s  kernel {kms:.3f} ms", file=sys.stderr, flush=True)
    del outs
    torch.cuda.empty_cache()

    det = {n: r for n, r in results.items() if not n.startswith("atomic")}
    atom = {n: r for n, r in results.items() if n.startswith("atomic")}
    best = max(det, key=lambda n: det[n]["tflops"])
    best_atomic = max(atom, key=lambda n: atom[n]["tflops"]) if atom else None
    value = det[best]["tflops"]
    ratio = value / atom[best_atomic]["tflops"] if best_atomic else None
    for r in results.values():
        r["pct_of_bf16_peak"] = 100.0 * r["tflops"] / PEAK_BF16_TFLOPS
        if best_atomic:
            r["ratio_vs_atomic"] = r["tflops"] / atom[best_atomic]["tflops"]

    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        try:
            from scheduling_persistent_fa_amd.profiling import kernel_source_digest
            c = json.load(open(PROFILE_COUNTERS))
            if (c.get("workload") == workload and c.get("schedule") == best
                    and c.get("kernel_source_sha256") == kernel_source_digest()):
                traffic = c.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None
    kt = det[best]["kernel_tflops"]
    sclk = det[best].get("sclk_ghz_est")
    return {
        "wl": wl,
        "value": value,
        "ms_per_step": det[best]["ms_per_step"],
        "config": {"workload": workload, "B": B, "Hq": Hq, "Hkv": Hkv, "S": S, "Sk": Sk, "D": D,
                   "mask": "causal" if causal else "full", "window": window, "tile": tile, "schedule": best,
                   "workgroups": info["num_cu"]},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "tflops_p10_p50_p90": [round(det[best][k], 2) for k in ("tflops_p10", "tflops_p50", "tflops_p90")],
        "sclk_ghz_est": None if sclk is None else round(sclk, 3),
        "ratio_vs_atomic": None if ratio is None else round(ratio, 4),
        "fastest_atomic": best_atomic,
        "roofline": {"bound": "mfma", "achieved": round(kt, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kt / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "bwd_kernel (persistent)", "kernel_ms": round(det[best]["kernel_ms"], 4)},
        "schedules": {n: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                      for n, r in results.items()},
    }


def block_bench(args):
    """Forward + backward of one synthetic transformer layer around the attention op.

    Llama-3-8B-shaped (hidden 4096, 32 query heads, 8 key/value heads, head dim
    128, SwiGLU MLP 14336), one sequence of 8192 tokens, causal, random-init
    weights, bf16.  The layer's matrix products are plain torch 2-D products;
    attention forward and backward are the library's.  Timed with the
    deterministic backward (adaptive schedule) and with the atomic one, to show
    the block-level share of the backward difference.
    """
    import torch
    from scheduling_persistent_fa_amd.attention import ATOMIC, AUTO
    from scheduling_persistent_fa_amd.autograd import dash_attention

    S, hidden, Hq, Hkv, D, ffn = 8192, 4096, 32, 8, 128, 14336
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(0)
    def w(i, o):
        return (torch.randn(i, o, device="cuda", generator=g) / math.sqrt(i)).to(torch.bfloat16).requires_grad_(True)
    Wqkv, Wo, W1, W3, W2 = w(hidden, (Hq + 2 * Hkv) * D), w(Hq * D, hidden), w(hidden, ffn), w(hidden, ffn), w(ffn, hidden)
    x = torch.randn(S, hidden, device="cuda", generator=g).to(torch.bfloat16).requires_grad_(True)

    def heads(t, h):  # [S, h*D] -> [1, h, S, D] contiguous
        return t.view(S, h, D).transpose(0, 1).contiguous().unsqueeze(0)

    def step(schedule):
        qkv = torch.mm(x, Wqkv)
        q = heads(qkv[:, :Hq * D], Hq)
        k = heads(qkv[:, Hq * D:(Hq + Hkv) * D], Hkv)
        v = heads(qkv[:, (Hq + Hkv) * D:], Hkv)
        a = dash_attention(q, k, v, causal=True, schedule=schedule)
        a2 = a.squeeze(0).transpose(0, 1).reshape(S, Hq * D)
        h = x + torch.mm(a2, Wo)
        m = torch.mm(torch.nn.functional.silu(torch.mm(h, W1)) * torch.mm(h, W3), W2)
        out = h + m
        out.float().square().mean().backward()

    res = {}
    for name, sched in (("deterministic", AUTO), ("atomic", ATOMIC)):
        for _ in range(args.warmup):
            step(sched)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(sched)
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / args.steps * 1e3
        print(f"[bench] block {name}: {res[name]:.3f} ms/step", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "transformer-layer fwd+bwd time with the library's attention (1 GPU)",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3_8b_shaped_layer_s8192", "S": S, "hidden": hidden, "Hq": Hq, "Hkv": Hkv,
                   "D": D, "ffn": ffn, "mask": "causal"},
        "ms_per_step": {k: round(v, 4) for k, v in res.items()},
        "block_speedup_det_vs_atomic": round(res["atomic"] / res["deterministic"], 4),
    }), flush=True)


if __name__ == "__main__":
    main()
