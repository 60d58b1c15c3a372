"""Build libdash_attn.so in-tree with hipcc for gfx950.

``python -m scheduling_persistent_fa_amd.build`` compiles the HIP kernels, the
C ABI and the host scheduler into ``scheduling_persistent_fa_amd/libdash_attn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdash_attn.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for device code (a host-pass warning
# about the unknown feature is expected and harmless).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    sources = [os.path.join(CSRC, f) for f in ("kernels.hip", "noalloc.hip", "api.cpp", "schedule.cpp")]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wshadow", "-Wno-unused-function", *DEVICE_FLAGS, "-o", tmp, *sources,
           "-lrocprofiler-sdk-roctx"]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose or resource_usage:
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


def resource_table() -> str:
    """Markdown table of the compiler's resource use per kernel of kernels.hip
    (registers, scratch spill, LDS, occupancy), from
    -Rpass-analysis=kernel-resource-usage on a device-only compile."""
    import re
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           *DEVICE_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-o", os.devnull, os.path.join(CSRC, "kernels.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    rows, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+(.*?): (.*?) \[-Rpass-analysis", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = {"name": val}
            rows.append(cur)
        elif cur is not None:
            cur[key] = val
    names = [r_["name"] for r_ in rows]
    cxxfilt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    if cxxfilt:
        out = subprocess.run([cxxfilt], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
        for r_, n in zip(rows, out):
            r_["name"] = n.replace("dash::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    cols = ["VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "VGPRs Spill", "LDS Size [bytes/block]",
            "Occupancy [waves/SIMD]"]
    lines = ["| kernel | " + " | ".join(cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for r_ in rows:
        lines.append(f"| `{r_['name']}` | " + " | ".join(r_.get(c, "") for c in cols) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    if "--resource-table" in sys.argv:
        print(resource_table())
    else:
        build(verbose=True, resource_usage="--resource-usage" in sys.argv)
