"""Build libtopk.so and libtopk_probe.so (HIP, gfx950) in-tree with hipcc.

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
SCORE_SRC = os.path.join(PKG, "csrc", "score.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtopk.so")
PROBE_SRC = os.path.join(PKG, "csrc", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "libtopk_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB, extra=(), src=(SRC, SCORE_SRC)) -> list[str]:
    srcs = [src] if isinstance(src, str) else list(src)
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed FP32: keep the backend from forming packed FP32 ops
        # (the selection's floating point only sizes the work; the scorer's
        # epilogue is scalar FP32 FMAs and roundings to BF16)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # every wave-level atomic here is already issued by one lane with the
        # wave's total; the backend's own aggregation would only add work
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        # the scorer's matrix-core results land in VGPRs, where its epilogue
        # reads them, instead of AGPRs copied out one by one (the selection
        # has no MFMA: its code is the same either way)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, *extra, "-o", out, *srcs,
    ]


def _build_one(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = command(tmp, src=src)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _build_one(PROBE_SRC, PROBE_LIB, verbose)
    return _build_one((SRC, SCORE_SRC), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
