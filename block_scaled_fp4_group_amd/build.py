"""Build the gfx950 shared library in-tree with hipcc (no torch involved).

    python -m block_scaled_fp4_group_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoefp4.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def command(out: str = LIB) -> list:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            *srcs, "-o", out]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
