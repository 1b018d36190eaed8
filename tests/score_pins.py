"""Pins of the FP8 and MXFP4 MQA indexer logits oracle
(oracle/score_oracle.c): facts fixed outside the oracle -- library routines
(torch's FP8 E4M3 decode, its float32 -> bfloat16 rounding, an FP32 matmul
on inputs whose sums it holds exactly), the E2M1 format's value table
(tests/golden/e2m1_values.txt), closed forms, invariants of the tolerance
interval, the hand-worked cases of tests/golden/mqa_worked.txt, and the
reduction of MXFP4 inputs whose scales are powers of two shared by a whole
dot product to the FP8 path (pinned on its own).

Run as a script with a library path, it applies every pin to that library
and exits non-zero when one fails (the planted-mistake tests do this).
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "mqa_worked.txt")
E2M1_TABLE = os.path.join(HERE, "golden", "e2m1_values.txt")
HEADS, DIM = 32, 128


def _torch():
    import torch
    return torch


def _bf16_bits_of_f32(x):
    """torch's float32 -> bfloat16 conversion (round to nearest, ties to
    even), as patterns."""
    torch = _torch()
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _f32_of_bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def narrow_e4m3(rng, shape):
    """E4M3 bytes of magnitude 0.5 .. 7.5 (exponent fields 6..9) or zero:
    the products are multiples of 2^-8 below 2^6, so any sum of 128 of them
    is exact in FP32."""
    b = (rng.integers(0, 2, shape, dtype=np.uint8) << 7) | (0x30 + rng.integers(0, 32, shape, dtype=np.uint8))
    z = rng.random(shape) < 0.1
    return np.where(z, np.uint8(0), b).astype(np.uint8)


def full_e4m3(rng, shape):
    """Any E4M3 byte but the two NaNs."""
    b = rng.integers(0, 256, shape, dtype=np.uint8)
    return np.where((b & 0x7F) == 0x7F, b ^ 0x01, b).astype(np.uint8)


def pin_e4m3_by_torch(so):
    """Every E4M3 byte decodes as torch's float8_e4m3fn does (NaN at the
    same two codes)."""
    torch = _torch()
    codes = np.arange(256, dtype=np.uint8)
    v = so.e4m3(codes)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(v), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(v[ok], t[ok])
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9


def pin_bf16_round_by_torch(so):
    """Rounding to BF16 agrees with torch's float32 -> bfloat16 conversion
    on random values and on exact ties (half way between two BF16 values,
    where the even one wins)."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    base = _f32_of_bf16(rng.integers(0x0080, 0x7F00, 2000).astype(np.uint16))
    ties = (base.astype(np.float64) * (1 + 2.0 ** -8)).astype(np.float32)   # exact midpoints
    ties = np.concatenate([ties, -ties])
    for arr in (x, ties):
        assert np.array_equal(so.bf16_round(arr.astype(np.float64)), _bf16_bits_of_f32(arr))


def _single_head_inputs(rng, h):
    q = np.zeros((HEADS, DIM), np.uint8)
    q[h] = narrow_e4m3(rng, DIM)
    key = narrow_e4m3(rng, DIM)
    w = np.zeros(HEADS, np.uint16)
    w[h] = 0x3F80
    return q, w, key


def pin_single_head_by_torch(so):
    """One head with weight 1 and the others 0: the logit is bf16(relu(q .
    key)) times the scale, with the dot product from torch's FP32 matmul
    (exact on these inputs)."""
    torch = _torch()
    rng = np.random.default_rng(12)
    for trial in range(64):
        h = int(rng.integers(0, HEADS))
        q, w, key = _single_head_inputs(rng, h)
        s = int(rng.integers(120, 135))
        qf = torch.from_numpy(q[h].copy()).view(torch.float8_e4m3fn).float()
        kf = torch.from_numpy(key.copy()).view(torch.float8_e4m3fn).float()
        d = torch.relu(qf @ kf).to(torch.bfloat16).float() * 2.0 ** (s - 127)
        want = int(d.to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        ex, lo, hi = so.mqa_logit(q, w, key, s)
        assert ex == want and lo == ex and hi == ex, (trial, hex(ex), hex(want))


def pin_sum_of_ones(so):
    """Every head's value 1 and every weight 1: each accumulator counts to
    8 exactly, the logit is 32 (0x4200), and zero weights give +0."""
    q = np.zeros((HEADS, DIM), np.uint8)
    q[:, 0] = 0x38
    key = np.zeros(DIM, np.uint8)
    key[0] = 0x38
    assert so.mqa_logit(q, np.full(HEADS, 0x3F80, np.uint16), key, 127)[0] == 0x4200
    assert so.mqa_logit(q, np.zeros(HEADS, np.uint16), key, 127)[0] == 0x0000


def _parse_bytes(spec):
    out = {}
    for item in spec.split(","):
        d, b = item.split("=")
        out[int(d)] = int(b, 16)
    return out


def golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, kspec, qspec, wspec, s, want = [x.strip() for x in line.split("|")]
        key = np.zeros(DIM, np.uint8)
        for d, b in _parse_bytes(kspec).items():
            key[d] = b
        q = np.zeros((HEADS, DIM), np.uint8)
        for part in qspec.split(";"):
            h, dims = part.split(":", 1)
            for d, b in _parse_bytes(dims).items():
                q[int(h), d] = b
        w = np.zeros(HEADS, np.uint16)
        if wspec.startswith("all="):
            w[:] = int(wspec[4:], 16)
        else:
            for h, b in _parse_bytes(wspec).items():
                w[h] = b
        cases.append((name, q, w, key, int(s, 16), int(want, 16)))
    return cases


def pin_worked_cases(so):
    """The hand-worked logits: chain order, accumulator pairing, relu,
    scale, negative weights, and the head value taken as FP32 first."""
    cases = golden_cases()
    assert len(cases) == 7
    for name, q, w, key, s, want in cases:
        ex, lo, hi = so.mqa_logit(q, w, key, s)
        assert ex == want, (name, hex(ex), hex(want))
        assert lo == ex and hi == ex, name


def _value_key(bits):
    """Order of BF16 values as unsigned keys (negatives inverted)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32)
    return np.where(b & 0x8000, b ^ 0xFFFF, b ^ 0x8000)


def pin_interval(so):
    """The tolerance interval: with delta 0 on inputs whose FP32 sums are
    exact it is the single exact value; with delta 2^-10 on full-range
    inputs and weights of both signs it always holds the exact value, is
    wider than a point somewhere, and grows with delta."""
    rng = np.random.default_rng(13)
    rows, nk = 3, 24
    q = narrow_e4m3(rng, (rows, HEADS, DIM))
    keys = narrow_e4m3(rng, (nk, DIM))
    w = _bf16_bits_of_f32(rng.standard_normal((rows, HEADS)).astype(np.float32) * 0.3)
    sc = rng.integers(118, 136, nk).astype(np.uint8)
    ex, lo, hi = so.mqa_logits(q, w, keys, sc, 0.0)
    assert np.array_equal(lo, ex) and np.array_equal(hi, ex)
    qf = full_e4m3(rng, (rows, HEADS, DIM))
    kf = full_e4m3(rng, (nk, DIM))
    kf[:, 64:] = 0                                          # keep logits finite
    qf[:, :, 64:] = 0
    ex, lo, hi = so.mqa_logits(qf, w, kf, np.full(nk, 100, np.uint8), 2.0 ** -10)
    ke, kl, kh = _value_key(ex), _value_key(lo), _value_key(hi)
    assert np.all(kl <= ke) and np.all(ke <= kh)
    assert np.any(kl < kh)
    _, lo2, hi2 = so.mqa_logits(qf, w, kf, np.full(nk, 100, np.uint8), 2.0 ** -6)
    assert np.all(_value_key(lo2) <= kl) and np.all(_value_key(hi2) >= kh)


def e2m1_table():
    """{code: value} from tests/golden/e2m1_values.txt."""
    out = {}
    for line in open(E2M1_TABLE):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, value = line.split()[:2]
        out[int(code, 16)] = float(value)
    assert len(out) == 16
    return out


def _e4m3_byte_of(value):
    """The E4M3 byte of an exactly representable value, found through
    torch's float8_e4m3fn decode (not the oracle's)."""
    torch = _torch()
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    hit = np.nonzero((vals == value) & ~np.isnan(vals) & (np.signbit(vals) == np.signbit(value)))[0]
    assert hit.size == 1, value
    return np.uint8(hit[0])


def _fp8_of_fp4(rows_of_nibbles):
    """E2M1 bytes [..., 64] (low nibble first) as E4M3 bytes [..., 128] of
    the same values."""
    table = e2m1_table()
    lut = np.array([_e4m3_byte_of(table[c]) for c in range(16)], np.uint8)
    b = np.asarray(rows_of_nibbles, np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = lut[b & 15]
    out[..., 1::2] = lut[b >> 4]
    return out


def pin_e2m1_by_format_table(so):
    """Every E2M1 code decodes to the value the format's definition gives
    (the golden table), and each of those values is an E4M3 value under
    torch's decode."""
    table = e2m1_table()
    v = so.e2m1(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert v[c] == table[c] and np.signbit(v[c]) == np.signbit(table[c]), (c, v[c], table[c])
        _e4m3_byte_of(table[c])


def pin_mxfp4_nibble_order(so):
    """Closed form: a byte's two nibbles are two dims.  A key holding 6 in
    the high nibble of byte 0 against a head holding 1 in the same nibble
    (weight 1, all scales 1) gives 6 (0x40C0); the head's 1 in the other
    nibble gives +0.  (Which nibble is the even dim cannot change a logit:
    the query and the key share the order, and a byte never straddles two
    scale blocks.)"""
    q = np.zeros((HEADS, DIM // 2), np.uint8)
    qs = np.full((HEADS, 4), 127, np.uint8)
    key = np.zeros(DIM // 2, np.uint8)
    ks = np.full(4, 127, np.uint8)
    w = np.zeros(HEADS, np.uint16)
    w[0] = 0x3F80
    key[0] = 0x70   # dim 1: code 7 (6.0); dim 0: code 0
    q[0, 0] = 0x20  # dim 1: code 2 (1.0)
    assert so.mxfp4_logit(q, qs, w, key, ks)[0] == 0x40C0
    q[0, 0] = 0x02  # dim 0: code 2
    assert so.mxfp4_logit(q, qs, w, key, ks)[0] == 0x0000


def _random_fp4(rng, shape):
    return rng.integers(0, 256, shape, dtype=np.uint8)


def pin_mxfp4_unit_scales_equal_fp8(so):
    """With every scale 1 (byte 127) an MXFP4 logit is the FP8 logit of the
    same values (E4M3 bytes by torch's decode, key scale 127): exact value
    and tolerance interval alike."""
    rng = np.random.default_rng(21)
    for trial in range(24):
        q4 = _random_fp4(rng, (HEADS, DIM // 2))
        k4 = _random_fp4(rng, (DIM // 2,))
        w = _bf16_bits_of_f32(rng.standard_normal(HEADS).astype(np.float32) * 0.5)
        qs = np.full((HEADS, 4), 127, np.uint8)
        ks = np.full(4, 127, np.uint8)
        for delta in (0.0, 2.0 ** -20, 2.0 ** -10):
            a = so.mxfp4_logit(q4, qs, w, k4, ks, delta)
            b = so.mqa_logit(_fp8_of_fp4(q4), w, _fp8_of_fp4(k4), 127, delta)
            a = tuple(0 if x == 0x8000 else x for x in a)
            b = tuple(0 if x == 0x8000 else x for x in b)
            assert a == b, (trial, delta, [hex(x) for x in a], [hex(x) for x in b])


def pin_mxfp4_block_scales(so):
    """Closed form: when only block b of the key holds values and every
    head's scale of block b is the same sq, the two scales act as one power
    of two on each dot product, so the logit is the FP8 logit of the same
    values with the key scale byte sq + sk - 127 (the other blocks' scales
    are then irrelevant)."""
    rng = np.random.default_rng(22)
    for trial in range(32):
        b = trial % 4
        q4 = _random_fp4(rng, (HEADS, DIM // 2))
        k4 = np.zeros(DIM // 2, np.uint8)
        k4[16 * b:16 * b + 16] = _random_fp4(rng, (16,))
        w = _bf16_bits_of_f32(rng.standard_normal(HEADS).astype(np.float32) * 0.5)
        qs = rng.integers(100, 155, (HEADS, 4)).astype(np.uint8)
        sq = int(rng.integers(110, 145))
        qs[:, b] = sq
        ks = rng.integers(100, 155, 4).astype(np.uint8)
        sk = int(rng.integers(110, 145))
        ks[b] = sk
        a = so.mxfp4_logit(q4, qs, w, k4, ks)[0]
        f = so.mqa_logit(_fp8_of_fp4(q4), w, _fp8_of_fp4(k4), sq + sk - 127)[0]
        assert (0 if a == 0x8000 else a) == (0 if f == 0x8000 else f), (trial, hex(a), hex(f))


def pin_mxfp4_interval(so):
    """The MXFP4 tolerance interval: a point with delta 0; with delta 2^-20
    on block scales 120..134 it holds the exact value and grows with delta."""
    rng = np.random.default_rng(23)
    rows, nk = 2, 16
    q = _random_fp4(rng, (rows, HEADS, DIM // 2))
    qs = rng.integers(120, 135, (rows, HEADS, 4)).astype(np.uint8)
    w = _bf16_bits_of_f32(rng.standard_normal((rows, HEADS)).astype(np.float32) * 0.5)
    keys = _random_fp4(rng, (nk, DIM // 2))
    ks = rng.integers(120, 135, (nk, 4)).astype(np.uint8)
    ex, lo, hi = so.mxfp4_logits(q, qs, w, keys, ks, 0.0)
    assert np.array_equal(lo, ex) and np.array_equal(hi, ex)
    widths = []
    for delta in (2.0 ** -20, 2.0 ** -12, 2.0 ** -6):
        e2, l2, h2 = so.mxfp4_logits(q, qs, w, keys, ks, delta)
        assert np.array_equal(e2, ex)
        kl, ke, kh = _value_key(l2), _value_key(e2), _value_key(h2)
        assert np.all(kl <= ke) and np.all(ke <= kh)
        widths.append(int((kh - kl).sum()))
    assert widths[0] <= widths[1] <= widths[2] and widths[2] > 0, widths


ALL_PINS = [pin_e4m3_by_torch, pin_bf16_round_by_torch, pin_single_head_by_torch,
            pin_sum_of_ones, pin_worked_cases, pin_interval, pin_e2m1_by_format_table,
            pin_mxfp4_nibble_order, pin_mxfp4_unit_scales_equal_fp8, pin_mxfp4_block_scales,
            pin_mxfp4_interval]


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    from oracle.score import ScoreOracle
    so = ScoreOracle(sys.argv[1])
    failed = 0
    for pin in ALL_PINS:
        try:
            pin(so)
        except Exception as e:  # noqa: BLE001 - report every failing pin
            failed += 1
            print(f"{pin.__name__}: {type(e).__name__} {e}")
    sys.exit(1 if failed else 0)
