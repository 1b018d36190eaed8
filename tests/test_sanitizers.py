"""Sanitizer builds on the CPU: the oracle's C source under gcc's
AddressSanitizer and UndefinedBehaviorSanitizer, and libtopk's host code
(argument checks, error reporting) under clang's, each driven by a small
program in tests/sanitize/.  No GPU is used: the device code is compiled
but never launched, and every call the host driver makes is rejected (or
has nothing to do) before any GPU work."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
                    os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "topk_oracle.c"), "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe])
    assert rc == 0 and "oracle driver done" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_score_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "score_driver")
    rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
                    os.path.join(HERE, "score_driver.c"),
                    os.path.join(ROOT, "oracle", "score_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe])
    assert rc == 0 and "score driver done" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_host_checks_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libtopk_san.so")
    exe = str(tmp_path / "host_driver")
    inc = os.path.join(ROOT, "include")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-O2", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                    "-I", inc, "-o", lib,
                    os.path.join(ROOT, "exact_row_wise_amd", "csrc", "libtopk.hip"),
                    os.path.join(ROOT, "exact_row_wise_amd", "csrc", "score.hip")])
    assert rc == 0, log
    rc, log = _run([HIPCC, "-O1", "-g", "-std=c++17", *san[:4], "-I", inc, "-o", exe,
                    os.path.join(HERE, "host_driver.cpp"), "-L", str(tmp_path), "-ltopk_san",
                    "-Wl,-rpath," + str(tmp_path)])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime's own at exit
    rc, log = _run([exe], env=env)
    assert rc == 0 and "host driver: 0 failure(s)" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
