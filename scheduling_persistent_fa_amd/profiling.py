"""Summaries of rocprofv3 output for profiles/.

``python -m scheduling_persistent_fa_amd.profiling stats DIR OUT.md "COMMAND"``
    writes a kernel-time table from DIR/*kernel_stats.csv.
``python -m scheduling_persistent_fa_amd.profiling traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
        COPY_BYTES WORKLOAD SCHEDULE OUT.json``
    turns FETCH_SIZE / WRITE_SIZE counter runs of the backward kernel into HBM
    bytes per launch, each scaled by what the same counter reads for a plain
    copy of COPY_BYTES, and records the kernel-source digest they belong to.
``python -m scheduling_persistent_fa_amd.profiling counters OUT.md "COMMANDS" DIR [DIR ...]``
    writes the per-dispatch median of every counter of the backward kernel
    found in the DIRs (one rocprofv3 --pmc pass each), with a few ratios.
``python -m scheduling_persistent_fa_amd.profiling power OUT.md INTERVAL_S -- COMMAND ...``
    runs COMMAND as a child process and samples the socket power and the
    graphics clock of every chiplet with ``amd-smi metric -p -c`` every
    INTERVAL_S seconds while it runs.
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


def _all_counters(prof_dir: str, name_filter: str):
    per = {}
    for r in csv.DictReader(open(_one(os.path.join(prof_dir, "**", "*counter_collection.csv")))):
        if name_filter in r["Kernel_Name"]:
            d = per.setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: statistics.median(v.values()) for k, v in per.items()}


# Ratios reported when their counters exist.  GRBM_GUI_ACTIVE is summed over
# the 8 chiplets (XCDs), so kernel cycles = GRBM_GUI_ACTIVE / 8; the SQ busy and
# LDS counters are summed over the 1024 SIMDs or the 256 CUs, the TCP counter
# over the 256 CUs.  (label, numerator, units the numerator is summed over)
_PER_KERNEL_CYCLE = [
    ("MFMA busy, share of SIMD cycles", "SQ_VALU_MFMA_BUSY_CYCLES", 1024),
    ("LDS indexed-access active, share of CU cycles", "SQ_LDS_IDX_ACTIVE", 256),
    ("LDS bank-conflict stall, share of CU cycles", "SQ_LDS_BANK_CONFLICT", 256),
    ("TCP pending stall, share of CU cycles", "TCP_PENDING_STALL_CYCLES", 256),
]


def counters_table(out_md: str, commands: str, dirs) -> None:
    vals = {}
    for d in dirs:
        vals.update(_all_counters(d, BWD_KERNEL))
    lines = [f"# Hardware counters of the persistent backward kernel — `{os.path.basename(out_md)}`", "",
             "Commands (one counter pass per run):", "", "```", commands, "```", "",
             "Median per dispatch of the backward kernel:", "", "| counter | value |", "|---|---|"]
    for k in sorted(vals):
        lines.append(f"| {k} | {vals[k]:.4g} |")
    lines += ["", "| ratio | value |", "|---|---|"]
    if vals.get("GRBM_GUI_ACTIVE", 0) > 0:
        cycles = vals["GRBM_GUI_ACTIVE"] / 8
        lines.append(f"| kernel cycles (GRBM_GUI_ACTIVE / 8) | {cycles:.4g} |")
        for label, num, units in _PER_KERNEL_CYCLE:
            if num in vals:
                lines.append(f"| {label} | {vals[num] / (cycles * units):.3f} |")
    if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_LDS_IDX_ACTIVE", 0) > 0:
        lines.append(f"| LDS bank-conflict cycles per LDS-active cycle | "
                     f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_LDS_IDX_ACTIVE']:.3f} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and vals.get("SQ_INSTS_MFMA", 0) > 0:
        lines.append(f"| MFMA busy cycles per MFMA instruction | "
                     f"{vals['SQ_VALU_MFMA_BUSY_CYCLES'] / vals['SQ_INSTS_MFMA']:.1f} |")
    if "TCC_HIT" in vals and "TCC_MISS" in vals:
        lines.append(f"| L2 hit rate | {vals['TCC_HIT'] / (vals['TCC_HIT'] + vals['TCC_MISS']):.3f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def power_samples(out_md: str, interval: float, cmd: list) -> int:
    """Socket power and per-chiplet graphics clocks while ``cmd`` runs (amd-smi text output)."""
    import re
    import subprocess
    import time
    child = subprocess.Popen(cmd)
    rows = []
    t0 = time.time()
    while child.poll() is None:
        time.sleep(interval)
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=60)
        pw = re.search(r"SOCKET_POWER: (\d+(?:\.\d+)?) W", r.stdout)
        clks = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK: (\d+) MHz", r.stdout)]
        if pw and clks:
            rows.append((time.time() - t0, float(pw.group(1)), clks))
    rc = child.wait()
    peak = max((w for _, w, _ in rows), default=0.0)
    loaded = [(w, c) for _, w, c in rows if w >= 0.5 * peak]
    lines = [f"# Socket power and graphics clocks — `{os.path.basename(out_md)}`", "",
             "Command (the sampler runs the benchmark as a child process):", "", "```",
             f"python -m scheduling_persistent_fa_amd.profiling power {out_md} {interval:g} -- " + " ".join(cmd), "```", "",
             "| t (s) | socket power (W) | graphics clock per chiplet, min / mean / max (MHz) |", "|---|---|---|"]
    for t, w, c in rows:
        lines.append(f"| {t:.1f} | {w:.0f} | {min(c)} / {sum(c) / len(c):.0f} / {max(c)} |")
    if loaded:
        mw = sum(w for w, _ in loaded) / len(loaded)
        allc = [x for _, c in loaded for x in c]
        lines += ["", f"Under load ({len(loaded)} samples at 50 % or more of the highest power): "
                      f"mean socket power {mw:.0f} W, graphics clock {min(allc)}–{max(allc)} MHz "
                      f"(mean {sum(allc) / len(allc):.0f} MHz) over {len(loaded[0][1])} chiplets."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rc


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        counters_table(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif sys.argv[1] == "stats":
        stats_table(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    elif sys.argv[1] == "power":
        sep = sys.argv.index("--")
        sys.exit(power_samples(sys.argv[2], float(sys.argv[3]), sys.argv[sep + 1:]))
    else:
        raise SystemExit(__doc__)
