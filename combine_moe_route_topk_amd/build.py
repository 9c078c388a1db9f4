"""Build libmoe_dc.so in-tree with hipcc for gfx950.

Usage: python combine_moe_route_topk_amd/build.py [-v]
(run it as a script: importing the package first would load the old library).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_dc.so")
SOURCES = ["api.cpp", "route_topk.hip", "dispatch.hip", "combine.hip", "grouped_swiglu.hip",
           "grouped_gemm_fp8.hip", "gather_swiglu.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_dc.so)")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libmoe_dc.so next to this file."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
        "-I", os.path.join(HERE, "..", "include"),
    ]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc()] + common + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif lines and (verbose or any("warning" in l for l in lines)):
            print(f"[{src}]\n" + "\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{t}" for s, t in failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
