"""Seeded synthetic inputs for exact per-row BF16 top-k.

Shared by the tests, the smoke check and the benchmark.  This module holds
none of the selection arithmetic (no keys, no thresholds, no ordering): it
only draws BF16 bit patterns, valid lengths and block tables with numpy's
PCG64 generator.

The five workloads mirror the shapes and value mixes the pages describe for
decode-step indexer rows (vLLM ``decode_topk_cute`` module docstring: token
top-512 over BF16 logits, block top-2048 over 8-logit block maxima, crowded
rows of ~200 distinct values at 150K; sglang PR #39305 "Performance" and
"Accuracy": 16384-wide rows, k = 512, permuted block table with 64-token
pages, special bit patterns).  No real indexer logits are available, so
these stand in for them.

Every logit past a row's valid length is the poison pattern 0x7FFF (a
positive NaN, which would rank first) so that any read past the valid length
changes the result.
"""
from __future__ import annotations

import numpy as np

MODE_TOKEN = 0
MODE_BLOCK = 1
POISON = 0x7FFF
PAGE = 64

BF16_POS_INF = 0x7F80
BF16_NEG_INF = 0xFF80

# name -> (rows, width, k, mode)
CONFIGS = {
    1: dict(name="token_4x16384_k512", rows=4, width=16384, k=512, mode=MODE_TOKEN),
    2: dict(name="token_512x16384_ragged_k512_paged", rows=512, width=16384, k=512,
            mode=MODE_TOKEN),
    3: dict(name="token_64x150000_crowded_k512", rows=64, width=150000, k=512,
            mode=MODE_TOKEN),
    4: dict(name="block_64x1048576_k2048", rows=64, width=1048576, k=2048,
            mode=MODE_BLOCK),
    5: dict(name="token_8192x16384_k2048_edge", rows=8192, width=16384, k=2048,
            mode=MODE_TOKEN),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even of float32 to BF16 bit patterns.

    Keeps the sign of zero; NaN inputs become quiet NaNs with their sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> 16) & np.uint32(1)
    r = ((b + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (b >> 16) | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def _row_stride(width: int) -> int:
    return (width + 7) // 8 * 8


def _normal_bits(rng, shape, sigma=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def _poison_tail(logits: np.ndarray, valid_len: np.ndarray):
    for r in range(logits.shape[0]):
        v = int(valid_len[r])
        if v < logits.shape[1]:
            logits[r, max(v, 0):] = POISON


def _permuted_pages(rng, rows: int, width: int) -> np.ndarray:
    npages = (width + PAGE - 1) // PAGE
    pages = np.empty((rows, npages), dtype=np.int32)
    for r in range(rows):
        pages[r] = rng.permutation(npages).astype(np.int32)
    return pages


def _special_patterns() -> np.ndarray:
    """Signed zeros, smallest/largest denormals, infinities, quiet and
    signalling NaNs of both signs (BF16 bit patterns)."""
    return np.array([
        0x0000, 0x8000,          # +0, -0
        0x0001, 0x007F,          # smallest / largest positive denormal
        0x8001, 0x807F,          # the negative ones
        0x0080, 0x8080,          # smallest normals
        0x7F7F, 0xFF7F,          # largest finite
        0x7F80, 0xFF80,          # +inf, -inf
        0x7FC0, 0x7FFF, 0x7F81, 0x7FA5,   # +qNaN, +NaN max payload, +sNaN
        0xFFC0, 0xFFFF, 0xFF81, 0xFFA5,   # the negative ones
    ], dtype=np.uint16)


def _edge_row(rng, j: int, width: int) -> np.ndarray:
    """One of the saturation workload's special rows (kind j in 0..7)."""
    if j == 0:                                   # constant finite value
        while True:
            val = int(rng.integers(0, 1 << 16))
            if (val & 0x7F80) != 0x7F80:
                break
        return np.full(width, val, dtype=np.uint16)
    if j == 1:                                   # all -inf
        return np.full(width, BF16_NEG_INF, dtype=np.uint16)
    if j == 2:                                   # N(0,1) with 3000 +NaN
        row = _normal_bits(rng, width)
        pos = rng.choice(width, size=min(3000, width), replace=False)
        payload = rng.integers(1, 128, size=pos.size).astype(np.uint16)
        row[pos] = np.uint16(0x7F80) | payload
        return row
    if j == 3:                                   # +/-0 around the pivot
        row = np.where(rng.integers(0, 2, size=width) == 1, 0x8000, 0x0000).astype(np.uint16)
        npos = min(2047, width)
        pos = rng.choice(width, size=npos, replace=False)
        vals = np.abs(rng.standard_normal(npos, dtype=np.float32)) + np.float32(1e-3)
        row[pos] = f32_to_bf16_bits(vals)
        return row
    # full-range random bit patterns with injected special values
    row = rng.integers(0, 1 << 16, size=width, dtype=np.uint32).astype(np.uint16)
    spec = _special_patterns()
    nspec = min(width, 32 * spec.size)
    pos = rng.choice(width, size=nspec, replace=False)
    row[pos] = spec[np.arange(nspec) % spec.size]
    return row


def make(cfg: int, rows: int | None = None, width: int | None = None,
         seed: int | None = None, k: int | None = None) -> dict:
    """Inputs of workload ``cfg`` (1..5), optionally at a reduced size.

    Returns a dict with ``logits`` (uint16 [rows, row_stride]), ``valid_len``
    (int32 [rows]), ``k``, ``mode``, ``width``, ``row_stride``, ``pages``
    (int32 [rows, ceil(width/64)] or None), ``page_size`` and ``name``.
    """
    spec = CONFIGS[cfg]
    rows = spec["rows"] if rows is None else int(rows)
    width = spec["width"] if width is None else int(width)
    k = spec["k"] if k is None else int(k)
    mode = spec["mode"]
    seed = cfg if seed is None else int(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    stride = _row_stride(width)
    logits = np.full((rows, stride), POISON, dtype=np.uint16)
    valid_len = np.full(rows, width, dtype=np.int32)
    pages = None

    if cfg == 1:
        logits[:, :width] = _normal_bits(rng, (rows, width))
    elif cfg == 2:
        logits[:, :width] = _normal_bits(rng, (rows, width))
        nshort = max(1, rows // 10) if rows >= 2 else 0
        short = rng.permutation(rows)[:nshort]
        lo = min(k + 1, width)
        valid_len[:] = rng.integers(lo, width + 1, size=rows)
        valid_len[short] = rng.integers(1, min(k, width) + 1, size=nshort)
        pages = _permuted_pages(rng, rows, width)
    elif cfg == 3:
        levels = []
        seen = set()
        while len(levels) < 200:
            b = int(f32_to_bf16_bits(np.array([rng.standard_normal() * 2.0], np.float32))[0])
            if b not in seen:
                seen.add(b)
                levels.append(b)
        levels = np.array(levels, dtype=np.uint16)
        rank = rng.permutation(200)               # Zipf rank of each level
        w = 1.0 / (rank + 1.0)
        w /= w.sum()
        for r in range(rows):
            logits[r, :width] = levels[rng.choice(200, size=width, p=w)]
    elif cfg == 4:
        lo = min(16384, width)
        vl = rng.integers(lo, width + 1, size=rows)
        valid_len[:] = np.maximum(vl // 8 * 8, min(lo, width))
        for r in range(rows):
            row = _normal_bits(rng, width)
            nblk = width // 8
            ninf = int(round(0.01 * nblk))
            if ninf:
                blk = rng.choice(nblk, size=ninf, replace=False)
                row[:nblk * 8].reshape(nblk, 8)[blk] = BF16_NEG_INF
            logits[r, :width] = row
    elif cfg == 5:
        for r in range(rows):
            if r % 10 == 9:
                logits[r, :width] = _edge_row(rng, (r // 10) % 8, width)
            else:
                logits[r, :width] = _normal_bits(rng, width)
    else:
        raise ValueError(cfg)

    _poison_tail(logits, valid_len)
    return dict(name=spec["name"], cfg=cfg, logits=logits, valid_len=valid_len, k=k,
                mode=mode, width=width, row_stride=stride, pages=pages,
                page_size=PAGE if pages is not None else 0)


# ------------------------------------------------------------ scorer inputs
# The FP8 MQA indexer scorer's inputs (vLLM kimi_k3 indexer page, module
# docstring and IndexerScore): per query row 32 heads x 128 dims of FP8
# E4M3 and 32 BF16 head weights; per key 128 dims of FP8 E4M3 and a UE8M0
# scale byte; the rows of a request (qpr of them, the verify rows of one
# decode step) share its keys.  No trained query, weights or cache exist
# here, so the bytes are drawn directly: a sign, an exponent field and a
# mantissa per value (the generator decodes nothing).
SCORE_CONFIG = dict(name="score_fp8_64x150000_q1", requests=64, qpr=1, width=150000)
SCORE_FP4_CONFIG = dict(name="score_mxfp4_64x150000_q1", requests=64, qpr=1, width=150000)


def _e4m3_bytes(rng, shape, kind: str) -> np.ndarray:
    """E4M3 bytes: "narrow" exponent fields 6..9 (magnitudes 0.5 .. 7.5,
    whose products sum exactly in FP32) and about 10 % zeros; "wide" fields
    over 0..15, the sum of two uniform fields 0..7 and 0..8 (a quantized
    activation's spread, down to the subnormals), never the NaN code.  Two
    random bytes a value: sign and mantissa from the first, the exponent
    field from the second."""
    n = int(np.prod(shape))
    raw = np.frombuffer(rng.bytes(2 * n), np.uint8).reshape(2, n)
    sm = raw[0] & np.uint8(0x87)                      # sign and mantissa bits
    if kind == "narrow":
        exp = np.uint8(6) + (raw[1] & np.uint8(3))
        b = sm | (exp << 3)
        b = np.where(raw[1] >= np.uint8(230), np.uint8(0), b)
    else:
        exp = (raw[1] & np.uint8(7)) + ((raw[1] >> 3) % np.uint8(9))
        b = sm | (exp << 3)
        b = np.where((b & 0x7F) == 0x7F, b ^ np.uint8(1), b)
    return b.astype(np.uint8).reshape(shape)


def make_score(requests: int, qpr: int, width: int, kind: str = "wide", seed: int = 0,
               key_stride: int | None = None, ragged: bool = True) -> dict:
    """Seeded scorer inputs: q uint8 [rows, 32, 128], w BF16 patterns
    [rows, 32], keys uint8 [requests, key_stride, 128], key_scale uint8
    [requests, key_stride] (UE8M0 bytes 118..130), valid_len int32 [rows]
    (request r's length U[width / 2, width] when ragged, else width; its
    verify rows u = 0..qpr-1 see length - (qpr - 1 - u), clamped at 0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = requests * qpr
    ks = width if key_stride is None else key_stride
    q = _e4m3_bytes(rng, (rows, 32, 128), kind)
    keys = np.empty((requests, ks, 128), np.uint8)
    for r in range(requests):
        keys[r] = _e4m3_bytes(rng, (ks, 128), kind)
    key_scale = rng.integers(118, 131, (requests, ks), dtype=np.uint8)
    w = f32_to_bf16_bits(rng.standard_normal((rows, 32), dtype=np.float32) * np.float32(0.25))
    if ragged:
        lens = rng.integers(width // 2, width + 1, requests)
    else:
        lens = np.full(requests, width)
    vl = np.empty(rows, np.int32)
    for r in range(requests):
        for u in range(qpr):
            vl[r * qpr + u] = max(0, int(lens[r]) - (qpr - 1 - u))
    return dict(q=q, w=w, keys=keys, key_scale=key_scale, valid_len=vl, qpr=qpr, width=width,
                requests=requests, kind=kind)


def make_score_mxfp4(requests: int, qpr: int, width: int, kind: str = "blocks", seed: int = 0,
                     key_stride: int | None = None, ragged: bool = True) -> dict:
    """Seeded MXFP4 scorer inputs: q uint8 [rows, 32, 64] and keys uint8
    [requests, key_stride, 64] of random E2M1 nibbles (two a byte), q_scale
    uint8 [rows, 32, 4] and key_scale uint8 [requests, key_stride, 4] of
    UE8M0 bytes 120..134, w and valid_len as make_score.  kind "uniform":
    one scale for all four blocks of a head and of a key (each dot product
    then sums exactly in FP32); "blocks": a scale per 32-dim block."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = requests * qpr
    ks = width if key_stride is None else key_stride
    q = rng.integers(0, 256, (rows, 32, 64), dtype=np.uint8)
    keys = np.empty((requests, ks, 64), np.uint8)
    for r in range(requests):
        keys[r] = rng.integers(0, 256, (ks, 64), dtype=np.uint8)
    if kind == "uniform":
        q_scale = np.repeat(rng.integers(120, 135, (rows, 32, 1), dtype=np.uint8), 4, axis=2)
        key_scale = np.repeat(rng.integers(120, 135, (requests, ks, 1), dtype=np.uint8), 4, axis=2)
    elif kind == "blocks":
        q_scale = rng.integers(120, 135, (rows, 32, 4), dtype=np.uint8)
        key_scale = rng.integers(120, 135, (requests, ks, 4), dtype=np.uint8)
    else:
        raise ValueError(kind)
    w = f32_to_bf16_bits(rng.standard_normal((rows, 32), dtype=np.float32) * np.float32(0.25))
    if ragged:
        lens = rng.integers(width // 2, width + 1, requests)
    else:
        lens = np.full(requests, width)
    vl = np.empty(rows, np.int32)
    for r in range(requests):
        for u in range(qpr):
            vl[r * qpr + u] = max(0, int(lens[r]) - (qpr - 1 - u))
    return dict(q=q, q_scale=np.ascontiguousarray(q_scale), w=w, keys=keys,
                key_scale=np.ascontiguousarray(key_scale), valid_len=vl, qpr=qpr, width=width,
                requests=requests, kind=kind)
