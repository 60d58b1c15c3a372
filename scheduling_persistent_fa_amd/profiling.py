"""Summaries of rocprofv3 output for profiles/.

``python -m scheduling_persistent_fa_amd.profiling stats DIR OUT.md "COMMAND"``
    writes a kernel-time table from DIR/*kernel_stats.csv.
``python -m scheduling_persistent_fa_amd.profiling traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
        COPY_BYTES WORKLOAD SCHEDULE OUT.json``
    turns FETCH_SIZE / WRITE_SIZE counter runs of the backward kernel into HBM
    bytes per launch, each scaled by what the same counter reads for a plain
    copy of COPY_BYTES, and records the kernel-source digest they belong to.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(_HERE, "csrc", "kernels.hip")
BWD_KERNEL = "bwd_kernel<"


def kernel_source_digest() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _steady_average_us(prof_dir: str, name: str, skip: int):
    """Average duration of a kernel's dispatches after the first ``skip`` (warm-up) ones."""
    try:
        trace = _one(os.path.join(prof_dir, "**", "*kernel_trace.csv"))
    except FileNotFoundError:
        return None
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in csv.DictReader(open(trace))
            if r["Kernel_Name"] == name]
    durs = durs[skip:]
    return sum(durs) / len(durs) / 1e3 if durs else None


def stats_table(prof_dir: str, out_md: str, command: str, skip: int = 3) -> None:
    rows = list(csv.DictReader(open(_one(os.path.join(prof_dir, "**", "*kernel_stats.csv")))))
    lines = [f"# Kernel times — `{os.path.basename(out_md)}`", "", "Command:", "", "```", command, "```", "",
             f"`steady` averages the dispatches after the first {skip} of each kernel (the warm-up calls).", "",
             "| kernel | calls | average (us) | steady (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        steady = _steady_average_us(prof_dir, r["Name"], skip)
        name = r["Name"].replace("dash::(anonymous namespace)::", "").replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        st = f"{steady:.1f}" if steady is not None else "-"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {st} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _counter_per_dispatch(prof_dir: str, counter: str, name_filter: str):
    vals = {}
    for r in csv.DictReader(open(_one(os.path.join(prof_dir, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] == counter and name_filter in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, workload, schedule, out_json):
    copy_bytes = int(copy_bytes)
    kib = 1024.0
    # the copy kernel moves copy_bytes in and copy_bytes out per launch
    cf = statistics.median(_counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copy"))
    cw = statistics.median(_counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copy"))
    fetch_scale = copy_bytes / (cf * kib)
    write_scale = copy_bytes / (cw * kib)
    f = statistics.median(_counter_per_dispatch(fetch_dir, "FETCH_SIZE", BWD_KERNEL))
    w = statistics.median(_counter_per_dispatch(write_dir, "WRITE_SIZE", BWD_KERNEL))
    rec = {"workload": workload, "schedule": schedule, "kernel_source_sha256": kernel_source_digest(),
           "fetch_kib_raw": f, "write_kib_raw": w, "copy_fetch_scale": fetch_scale, "copy_write_scale": write_scale,
           "hbm_fetch_bytes_per_launch": f * kib * fetch_scale, "hbm_write_bytes_per_launch": w * kib * write_scale}
    rec["hbm_bytes_per_launch"] = rec["hbm_fetch_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    json.dump(rec, open(out_json, "w"), indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats_table(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    else:
        raise SystemExit(__doc__)
