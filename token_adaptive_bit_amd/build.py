"""Build libmbq.so (gfx950) in the package directory with hipcc.

Every translation unit is compiled for gfx950 only, with packed FP32 instructions
disabled (-packed-fp32-ops) and IEEE-correct float32 division.  The pack kernel is also
built with -ffp-contract=off: its float32 recursion must round every operation on its
own to reproduce the bit-exact MoBiSlice codes.

Usage:  python -m token_adaptive_bit_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmbq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = {
    "api.hip": [],
    "pack.hip": ["-ffp-contract=off"],
    "route.hip": [],
    "route_mlp.hip": [],
    "lowrank.hip": [],
    "decode.hip": [],
    "decode_stream.hip": [],
    "prefill.hip": [],
    "prefill_mfma.hip": [],
}

# Translation units whose kernels must not spill registers: their load pipelines rely on
# exact waits on the in-order memory counter, which spill traffic (scratch loads and
# stores) would stall, and the variants a launcher can pick are chosen to fit.  The build
# reads the compiler's resource-usage remarks and fails on any spill to scratch memory.
SPILL_FREE = ("decode_stream.hip", "prefill_mfma.hip", "route_mlp.hip", "lowrank.hip")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmbq)")


def _spills(remarks: str) -> list:
    """(kernel, vgpr spills, sgpr spills, scratch bytes) of every kernel that spills to memory."""
    out, name = [], None
    vals = {}
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name, vals = m.group(1), {}
            continue
        for key in ("VGPRs Spill", "SGPRs Spill", "ScratchSize \\[bytes/lane\\]"):
            m = re.search(" " + key + r": (\d+)", line)
            if m:
                vals[key[:5]] = int(m.group(1))
        if name and len(vals) == 3:
            if vals["VGPRs"] or vals["Scrat"]:  # SGPR spills into VGPR lanes touch no memory
                out.append((name, vals["VGPRs"], vals["SGPRs"], vals["Scrat"]))
            name = None
    return out


def _compile(src: str, extra: list, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    check = src in SPILL_FREE
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if check else []
    cmd = [hipcc(), *COMMON, *extra, *remarks, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if check:
        bad = _spills(res.stderr)
        if bad:
            lines = "\n".join(f"  {n}: {v} VGPR / {s} SGPR spills, {b} B scratch" for n, v, s, b in bad)
            raise RuntimeError(f"{src}: kernels spill registers:\n{lines}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
