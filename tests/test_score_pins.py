"""The FP8 and MXFP4 MQA logits oracle against its pins, and the pins against planted
mistakes (one-line changes to a temporary copy of oracle/score_oracle.c,
compiled on the CPU; every copy must fail at least one pin)."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle import score
from score_pins import ALL_PINS


@pytest.fixture(scope="module")
def so():
    return score.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(so, pin):
    pin(so)


# (description, exact text in score_oracle.c, replacement)
MUTANTS = [
    ("no relu", "r[h] = bf16r(fp32_round(d > 0 ? d : 0));", "r[h] = bf16r(fp32_round(d));"),
    ("head value not FP32 first", "r[h] = bf16r(fp32_round(d > 0 ? d : 0));",
     "r[h] = bf16r(d > 0 ? d : 0);"),
    ("heads in natural order", "const int h = j + 4 * i;", "const int h = 8 * j + i;"),
    ("accumulators paired 0+1, 2+3",
     "const long double t = bf16r(bf16r(a[0] + a[2]) + bf16r(a[1] + a[3]));",
     "const long double t = bf16r(bf16r(a[0] + a[1]) + bf16r(a[2] + a[3]));"),
    ("FMA not rounded", "a[j] = bf16r(r[h] * wh + a[j]);", "a[j] = r[h] * wh + a[j];"),
    ("E4M3 bias 8", "v = ldexpl(1.0L + m / 8.0L, e - 7);", "v = ldexpl(1.0L + m / 8.0L, e - 8);"),
    ("E4M3 subnormal step", "v = ldexpl((long double)m, -9);", "v = ldexpl((long double)m, -10);"),
    ("scale off by one", "ldexpl(1.0L, (int)scale - 127);", "ldexpl(1.0L, (int)scale - 128);"),
    ("ties away from zero", "nearbyintl(a / q) * q;", "roundl(a / q) * q;"),
    ("dot with the next dim", "oracle_e4m3(key[c]);", "oracle_e4m3(key[(c + 1) % DIM]);"),
    ("interval without delta", "const long double dl = d - (long double)delta * s, dh = d + (long double)delta * s;",
     "const long double dl = d, dh = d;"),
    ("negative weights keep bounds", "(wh >= 0 ? rlo[h] : rhi[h]) * wh + al[j];", "rlo[h] * wh + al[j];"),
    ("E2M1 bias 2", "v = ldexpl(1.0L + m / 2.0L, e - 1);", "v = ldexpl(1.0L + m / 2.0L, e - 2);"),
    ("E2M1 subnormal step", "v = m / 2.0L;", "v = m / 4.0L;"),
    ("blocks of 16 dims", "const int b = c / 32;", "const int b = c / 16 % 4;"),
    ("query scales ignored", "(int)q_scale[h * 4 + b] + (int)key_scale[b] - 254", "127 + (int)key_scale[b] - 254"),
    ("key scale of block 0 only", "(int)q_scale[h * 4 + b] + (int)key_scale[b] - 254", "(int)q_scale[h * 4 + b] + (int)key_scale[0] - 254"),
    ("MXFP4 scaled again after the sum", "logit_of_heads(dd, ss, w, delta, 1.0L, 1, exact, lo, hi);", "logit_of_heads(dd, ss, w, delta, 2.0L, 1, exact, lo, hi);"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, desc, old, new):
    src = open(score.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {desc}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path), str(tmp_path / "libmutant.so"), libs=("-lm",))
    pins = os.path.join(os.path.dirname(os.path.abspath(__file__)), "score_pins.py")
    res = subprocess.run([sys.executable, pins, lib], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, f"no pin catches the planted mistake: {desc}"
