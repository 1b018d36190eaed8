"""Build libtopk.so (HIP, gfx950) in-tree with hipcc.

    python -m exact_row_wise_amd.build        # or exact_row_wise_amd.build.build()
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "libtopk.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtopk.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=()) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed FP32 (the path has no floating point; keep the backend from
        # forming packed FP32 ops anywhere)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # every wave-level atomic here is already issued by one lane with the
        # wave's total; the backend's own aggregation would only add work
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, *extra, "-o", out, SRC,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
