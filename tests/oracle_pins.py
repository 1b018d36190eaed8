"""Pins of the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with what the pages or the mathematics fix:

* hand-worked values (``tests/golden/*.txt``, each file citing its passage);
* the order of the key against IEEE float order, exhaustively over all
  65,536 BF16 patterns (numpy float32 comparisons, not the key formula);
* brute force over every k-subset of tiny rows;
* numpy's own sort (a different sort from the oracle's qsort) for the k-th
  key and for the top-k values of NaN-free rows;
* closed forms (constant rows, short rows, -inf blocks, pinned newest block,
  clamped lengths) and the inverse-table round trip of the page transform.

The same pins are run against copies of the oracle built from deliberately
altered sources (``test_oracle_pins.py``), to show that a plausible mistake
anywhere in the oracle fails at least one of them.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOKEN, BLOCK = 0, 1


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _nan_mask(bits):
    return np.isnan(bf16_to_f32(bits))


# ---------------------------------------------------------------- key pins
def pin_key_fixed_points(orc):
    """Hand-worked keys (golden/key_fixed_points.txt)."""
    with open(os.path.join(GOLDEN, "key_fixed_points.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            b, k, what = line.split()[:3]
            got = int(orc.key(np.array([int(b, 16)], np.uint16))[0])
            assert got == int(k, 16), f"key({b}) = {got:#06x}, expected {k} ({what})"


def pin_key_bijection(orc):
    """The key is a bijection of the 16-bit patterns (ties only for equal bits)."""
    keys = orc.key(_all_patterns())
    assert np.array_equal(np.sort(keys), np.arange(1 << 16, dtype=np.uint16)), \
        "key is not a permutation of 0..65535"


def pin_key_follows_float_order(orc):
    """For every pair of non-NaN patterns: key order == IEEE value order,
    with -0 directly below +0 (the pages' value order)."""
    bits = _all_patterns()
    vals = bf16_to_f32(bits)
    ok = ~np.isnan(vals)
    b, v = bits[ok], vals[ok]
    positive_sign = (b & 0x8000) == 0        # breaks the +0 / -0 tie: -0 first
    order = np.lexsort((positive_sign, v))
    keys = orc.key(b[order]).astype(np.int64)
    assert np.all(np.diff(keys) > 0), "keys not strictly increasing in value order"


def pin_key_nan_placement(orc):
    """Positive NaNs above +inf, negative NaNs below -inf (reading of the
    pages: NaNs compare through the key like any pattern)."""
    bits = _all_patterns()
    keys = orc.key(bits).astype(np.int64)
    nan = _nan_mask(bits)
    neg = (bits & 0x8000) != 0
    finite_keys = keys[~nan]
    assert keys[nan & ~neg].min() > finite_keys.max(), "+NaN not above +inf"
    assert keys[nan & neg].max() < finite_keys.min(), "-NaN not below -inf"


def pin_is_nan(orc):
    """oracle_is_nan agrees with IEEE isnan on all patterns (sampled)."""
    bits = _all_patterns()
    ref = _nan_mask(bits)
    for b in list(range(0x7F70, 0x7F90)) + list(range(0xFF70, 0xFF90)) + [0, 0x8000, 0x7FFF, 0xFFFF]:
        assert orc.is_nan(b) == bool(ref[b]), f"is_nan({b:#06x})"


# ---------------------------------------------------------- block key pins
def pin_block_key_max(orc):
    """Non-NaN blocks without zeros: the block key is the key of the float
    maximum (numpy argmax over float values)."""
    rng = np.random.Generator(np.random.PCG64(11))
    for _ in range(400):
        bits = rng.integers(0, 1 << 16, size=8).astype(np.uint16)
        vals = bf16_to_f32(bits)
        if np.isnan(vals).any() or (vals == 0).any():
            continue
        mx = bits[int(np.argmax(vals))]
        assert orc.block_key(bits) == int(orc.key(np.array([mx], np.uint16))[0]), \
            f"block max of {bits}"


def pin_block_key_nan(orc):
    """A block holding a NaN of either sign, anywhere, is the canonical
    positive NaN (key 0xFFFF) -- the reading taken of NaN propagation."""
    rng = np.random.Generator(np.random.PCG64(12))
    for nanbits in (0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FFF, 0xFF81):
        for pos in range(8):
            bits = rng.integers(0x0000, 0x7F00, size=8).astype(np.uint16)
            bits[pos] = nanbits
            assert orc.block_key(bits) == 0xFFFF, f"NaN block {bits}"


def pin_block_key_special(orc):
    """Closed forms: all -inf -> key(-inf); +0 beats -0; all -0 -> key(-0)."""
    assert orc.block_key([0xFF80] * 8) == 0x007F
    assert orc.block_key([0x8000] * 7 + [0x0000]) == 0x8000
    assert orc.block_key([0x8000] * 8) == 0x7FFF
    assert orc.block_key([0xFF80] * 7 + [0xBF80]) == 0x407F     # -1.0 beats -inf


def pin_row_keys_block(orc):
    """Block rows: n = ceil(v/8), the newest block keyed as +inf whatever it
    holds, the others keyed from their 8 logits."""
    rng = np.random.Generator(np.random.PCG64(13))
    row = rng.integers(0, 1 << 16, size=64).astype(np.uint16)
    row[56:64] = 0xFF80                               # an all -inf block
    for v in (1, 7, 8, 9, 23, 24, 57, 64):
        keys = orc.row_keys(row, v, BLOCK)
        n = (v + 7) // 8
        assert keys.size == n, f"v={v}: n={keys.size}, expected {n}"
        assert keys[-1] == 0xFF80, f"v={v}: newest block not pinned"
        for b in range(n - 1):
            assert keys[b] == orc.block_key(row[8 * b:8 * b + 8]), f"v={v} block {b}"


# --------------------------------------------------------- selection pins
def _valid_topk_sets(keys, k):
    """All index sets S, |S| = k, with no unselected key above a selected one."""
    n = keys.size
    sets = []
    for S in itertools.combinations(range(n), k):
        sel = keys[list(S)]
        rest = np.delete(keys, list(S))
        if rest.size == 0 or sel.min() >= rest.max():
            sets.append(frozenset(S))
    return sets


def pin_bruteforce_tiny_rows(orc):
    """Every n <= 9, k < n: the oracle's index set is one of the valid top-k
    sets found by enumerating all k-subsets, in both modes."""
    rng = np.random.Generator(np.random.PCG64(14))
    alphabets = [
        None,                                               # any pattern
        np.array([0x3F80, 0xBF80, 0x0000, 0x8000], np.uint16),    # ties, +/-0
        np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x4000], np.uint16),  # NaN, inf
    ]
    for trial in range(90):
        n = 2 + trial % 8
        alpha = alphabets[trial % 3]
        if alpha is None:
            row = rng.integers(0, 1 << 16, size=n).astype(np.uint16)
        else:
            row = alpha[rng.integers(0, alpha.size, size=n)]
        keys = orc.row_keys(row, n, TOKEN)
        for k in range(1, n):
            out = orc.topk_row(row, n, k, TOKEN)
            valid = _valid_topk_sets(keys, k)
            assert frozenset(out.tolist()) in valid, f"token row {row}, k={k}: {out}"
    for trial in range(40):
        nb = 2 + trial % 6
        row = rng.integers(0, 1 << 16, size=8 * nb).astype(np.uint16)
        if trial % 2:
            row[rng.integers(0, 8 * nb, size=3)] = 0xFF80
            row[8 * (trial % (nb - 1)): 8 * (trial % (nb - 1)) + 8] = 0xFF80
        keys = orc.row_keys(row, 8 * nb, BLOCK)
        for k in range(1, nb):
            out = orc.topk_row(row, 8 * nb, k, BLOCK)
            sel = out[out >= 0]
            nneg = int((out < 0).sum())
            assert not (keys[sel] == 0x007F).any(), "a -inf block kept its index"
            # -1 entries stand for selected -inf blocks: complete the set with
            # the -inf blocks the row holds (any choice is equally valid).
            infb = [b for b in range(nb) if keys[b] == 0x007F and b not in sel]
            full = set(sel.tolist()) | set(infb[:nneg])
            assert len(full) == k, f"block row k={k}: {out}"
            assert frozenset(full) in _valid_topk_sets(keys, k), f"block row k={k}: {out}"


def pin_threshold_by_numpy_sort(orc):
    """numpy's sort gives the k-th key; the oracle's T, counts and selection
    agree: count(key > T) < k <= count(key >= T), selected >= T >= unselected."""
    rng = np.random.Generator(np.random.PCG64(15))
    for trial in range(30):
        n = int(rng.integers(20, 3000))
        k = int(rng.integers(1, n))
        if trial % 3 == 0:
            row = rng.integers(0, 1 << 16, size=n).astype(np.uint16)
        elif trial % 3 == 1:
            row = rng.choice(np.array([0x3F80, 0x4000, 0xBF80, 0x0000, 0x8000], np.uint16), n)
        else:
            row = rng.integers(0x3F00, 0x3F20, size=n).astype(np.uint16)
        keys = orc.row_keys(row, n, TOKEN)
        T_np = int(np.sort(keys)[n - k])
        res = orc.threshold(keys, k)
        assert res is not None
        T, gt, eq = res
        assert T == T_np, f"T {T:#x} != numpy {T_np:#x}"
        assert gt == int((keys > T).sum()) and eq == int((keys == T).sum())
        assert gt < k <= gt + eq
        out = orc.topk_row(row, n, k, TOKEN)
        sel = np.zeros(n, bool)
        sel[out] = True
        assert sel.sum() == k, "indices not distinct"
        assert keys[sel].min() >= T and (keys[~sel].max() if (~sel).any() else 0) <= T


def pin_values_match_numpy_topk(orc):
    """NaN-free, zero-free rows: the selected values are the k largest float
    values (numpy sort of float32), as a multiset."""
    rng = np.random.Generator(np.random.PCG64(16))
    for n, k in ((16384, 512), (16384, 2048), (5000, 700), (100, 99)):
        f = rng.standard_normal(n, dtype=np.float32)
        f[f == 0] = 1.0
        bits = ((f.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
        vals = bf16_to_f32(bits)
        assert not np.isnan(vals).any()
        out = orc.topk_row(bits, n, k, TOKEN)
        assert np.array_equal(np.sort(vals[out]), np.sort(vals)[n - k:]), f"n={n} k={k}"


# ------------------------------------------------------ closed-form pins
def pin_short_rows(orc):
    """n <= k: 0..n-1 in order then -1 (token); no logits consulted."""
    rng = np.random.Generator(np.random.PCG64(17))
    row = rng.integers(0, 1 << 16, size=100).astype(np.uint16)
    for v, k in ((0, 5), (1, 1), (5, 5), (5, 9), (100, 100), (37, 512)):
        out = orc.topk_row(row, v, k, TOKEN)
        exp = list(range(min(v, k))) + [-1] * (k - min(v, k))
        assert out.tolist() == exp, f"v={v} k={k}"


def pin_clamped_lengths(orc):
    """valid_len below 0 acts as 0, above the width as the width."""
    rng = np.random.Generator(np.random.PCG64(18))
    row = rng.integers(0, 0x7F00, size=40).astype(np.uint16)
    assert orc.topk_row(row, -5, 4, TOKEN).tolist() == [-1] * 4
    assert orc.topk_row(row, -5, 4, BLOCK).tolist() == [-1] * 4
    a = orc.topk_row(row, 1000, 7, TOKEN)
    b = orc.topk_row(row, 40, 7, TOKEN)
    assert sorted(a.tolist()) == sorted(b.tolist())


def pin_constant_row(orc):
    """A constant row: any k distinct indices (all keys equal)."""
    for bits in (0x3F80, 0xFF80, 0x8000, 0x7FC0):
        row = np.full(333, bits, np.uint16)
        out = orc.topk_row(row, 333, 100, TOKEN)
        assert len(set(out.tolist())) == 100 and out.min() >= 0 and out.max() < 333


def pin_block_neg_inf_rows(orc):
    """Block rows of -inf blocks: n > k gives the pinned newest block and
    k-1 entries of -1; n <= k gives -1 for every -inf block, the newest kept."""
    row = np.full(8 * 50, 0xFF80, np.uint16)
    out = orc.topk_row(row, 400, 10, BLOCK)
    assert sorted(out.tolist()) == [-1] * 9 + [49]
    out = orc.topk_row(row, 400, 60, BLOCK)
    assert out.tolist() == [-1] * 49 + [49] + [-1] * 10
    row[8 * 3] = 0x3F80                       # block 3 holds a 1.0
    out = orc.topk_row(row, 400, 2, BLOCK)
    assert sorted(out.tolist()) == [3, 49]


def pin_poison_not_selected(orc):
    """Logits past valid_len (poisoned with +NaN, the top key) never appear."""
    rng = np.random.Generator(np.random.PCG64(19))
    row = rng.integers(0, 0x7F00, size=512).astype(np.uint16)
    for v in (3, 100, 257, 511):
        row2 = row.copy()
        row2[v:] = 0x7FFF
        out = orc.topk_row(row2, v, 2, TOKEN)
        assert out.max() < v
        outb = orc.topk_row(row2, v, 2, BLOCK)
        assert outb.max() < (v + 7) // 8


def pin_page_transform_roundtrip(orc):
    """Inverting the permuted block table recovers the untransformed result."""
    rng = np.random.Generator(np.random.PCG64(20))
    width, P = 4096, 64
    pages = rng.permutation(width // P).astype(np.int32)
    inv = np.empty_like(pages)
    inv[pages] = np.arange(pages.size, dtype=np.int32)
    row = rng.integers(0, 0x7F00, size=width).astype(np.uint16)
    for v, k in ((4096, 512), (3000, 100), (77, 100)):
        plain = orc.topk_row(row, v, k, TOKEN)
        mapped = orc.topk_row(row, v, k, TOKEN, pages=pages, page_size=P)
        back = np.where(mapped >= 0, inv[np.maximum(mapped, 0) // P] * P + mapped % P, -1)
        assert np.array_equal(back, plain), f"v={v} k={k}"


def pin_worked_examples(orc):
    """Hand-worked rows (golden/worked_examples.txt)."""
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            if line.lstrip().startswith("#") or not line.strip():
                continue
            name, mode, v, k, P, pages, bits, kind, exp = [s.strip() for s in line.split("|")]
            mode = TOKEN if mode == "token" else BLOCK
            row = np.array([int(b, 16) for b in bits.split(",")], np.uint16)
            pg = None if pages == "-" else np.array([int(p) for p in pages.split(",")], np.int32)
            out = orc.topk_row(row, int(v), int(k), mode, pages=pg,
                               page_size=int(P) if pg is not None else 64)
            expected = [int(e) for e in exp.split(",")]
            if kind == "set":
                assert sorted(out.tolist()) == sorted(expected), f"{name}: {out.tolist()}"
            else:
                assert out.tolist() == expected, f"{name}: {out.tolist()}"


def _ordered_by_rank(keys, n, k):
    """The ordered selection straight from its definition: element i is taken
    when fewer than k elements come before it in the (key desc, index asc)
    order, i.e. (keys above it) + (equal keys at lower indices) < k; the taken
    indices are listed in ascending order.  No sort is involved."""
    sel = []
    for i in range(n):
        before = int((keys[:n] > keys[i]).sum()) + int((keys[:i] == keys[i]).sum())
        if before < k:
            sel.append(i)
    return sel


def pin_ordered_rank_definition(orc):
    """Ordered results of tiny rows (both modes, ragged and short lengths,
    tie-heavy and NaN/inf alphabets, with and without a block table) equal the
    rank definition bit for bit: ids ascending then -1, out mapped through the
    table with -inf blocks as -1, valid = min(n, k)."""
    rng = np.random.Generator(np.random.PCG64(33))
    alphabets = [
        None,
        np.array([0x3F80, 0xBF80, 0x0000, 0x8000], np.uint16),
        np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x4000], np.uint16),
    ]
    ps = 4
    for trial in range(120):
        mode = TOKEN if trial % 2 == 0 else BLOCK
        width = 8 * (1 + trial % 5)
        alpha = alphabets[trial % 3]
        if alpha is None:
            row = rng.integers(0, 1 << 16, size=width).astype(np.uint16)
        else:
            row = alpha[rng.integers(0, alpha.size, size=width)]
        if mode == BLOCK and trial % 4 == 1:
            row[0:8] = 0xFF80                                  # a -inf block
        v = int(rng.integers(0, width + 1))
        pages = rng.permutation((width + ps - 1) // ps).astype(np.int32) if trial % 3 == 0 else None
        keys = orc.row_keys(row, v, mode)
        n = keys.size
        for k in (1, 2, 3, 5, 9):
            out, ids, valid = orc.topk_ordered(row[None, :], [v], k, mode, pages=(
                None if pages is None else pages[None, :]), page_size=ps)
            sel = _ordered_by_rank(keys, n, k)
            want_ids = sel + [-1] * (k - len(sel))
            want_out = []
            for i in want_ids:
                o = i
                if i >= 0 and mode == BLOCK and keys[i] == 0x007F:
                    o = -1
                if o >= 0 and pages is not None:
                    o = int(pages[o // ps]) * ps + o % ps
                want_out.append(o)
            ctx = f"trial {trial} mode {mode} v {v} k {k}"
            assert int(valid[0]) == min(n, k), ctx
            assert ids[0].tolist() == want_ids, f"{ctx}: {ids[0]} vs {want_ids}"
            assert out[0].tolist() == want_out, f"{ctx}: {out[0]} vs {want_out}"


def pin_ordered_worked_cases(orc):
    """Hand-derived ordered results for the row 5, 7, 7, 3, 7 (token mode):
    the three 7s tie at the top, so k = 1 and 2 take the lowest-index 7s, k = 3
    all three, k = 4 adds the 5, and k = 6 is a short row."""
    row = np.array([0x40A0, 0x40E0, 0x40E0, 0x4040, 0x40E0, 0, 0, 0], np.uint16)
    want = {1: [1], 2: [1, 2], 3: [1, 2, 4], 4: [0, 1, 2, 4], 6: [0, 1, 2, 3, 4, -1]}
    for k, w in want.items():
        out, ids, valid = orc.topk_ordered(row[None, :], [5], k, TOKEN)
        assert out[0].tolist() == w and ids[0].tolist() == w, (k, out, ids)
        assert int(valid[0]) == min(5, k)
    # block mode: blocks (1, -inf, 9, 9) with the newest pinned: k = 2 takes
    # block 3 (pinned +inf) and the lowest-index 9 (block 2)
    b = np.zeros(32, np.uint16)
    b[0:8] = 0x3F80
    b[8:16] = 0xFF80
    b[16:24] = 0x4110
    b[24:32] = 0x4110
    out, ids, valid = orc.topk_ordered(b[None, :], [32], 2, BLOCK)
    assert ids[0].tolist() == [2, 3] and out[0].tolist() == [2, 3] and int(valid[0]) == 2
    out, ids, valid = orc.topk_ordered(b[None, :], [32], 4, BLOCK)
    assert ids[0].tolist() == [0, 1, 2, 3] and out[0].tolist() == [0, -1, 2, 3]

def _multirow_case(rng, rows, width, stride_pad, P, pstride_pad, mode):
    """A [rows, row_stride] matrix with row_stride > width (the padding holds
    the poison +NaN, the top key, and other rows' data would differ), ragged
    lengths (negative, zero, short, past the width) and a block table whose
    rows are longer than ceil(width / P)."""
    stride = width + stride_pad
    L = rng.integers(0, 1 << 16, size=(rows, stride)).astype(np.uint16)
    L[:, width:] = 0x7FFF
    lens = rng.integers(-3, width + 5, size=rows).astype(np.int32)
    lens[0], lens[-1] = width, 2
    npg = (width + P - 1) // P
    pages = rng.integers(0, 1000, size=(rows, npg + pstride_pad)).astype(np.int32)
    for r in range(rows):
        pages[r, :npg] = rng.permutation(npg) + 7 * r
    return L, lens, pages


def pin_multirow_driver(orc):
    """The multi-row drivers (oracle_topk_rows and oracle_topk_rows_ordered,
    with their host-thread split and row sub-selection) address row r at
    logits + r * row_stride, its table at pages + r * pages_stride and its
    outputs at r * k: each row of a multi-row call with row_stride > width,
    a table stride above ceil(width / P), ragged lengths and several threads
    equals the one-row call on that row alone (plain: the pinned one-row
    selection; ordered: the rank definition, which sorts nothing)."""
    rng = np.random.Generator(np.random.PCG64(34))
    for mode, width, k, P in ((TOKEN, 61, 9, 4), (BLOCK, 200, 7, 8), (TOKEN, 37, 40, 2)):
        rows = 11
        L, lens, pages = _multirow_case(rng, rows, width, 24, P, 5, mode)
        for threads in (1, 3):
            for pg in (None, pages):
                got = orc.topk(L, lens, k, mode, width=width, pages=pg, page_size=P,
                               threads=threads)
                for r in range(rows):
                    want = orc.topk_row(L[r, :width], int(lens[r]), k, mode,
                                        pages=None if pg is None else pg[r], page_size=P)
                    assert got[r].tolist() == want.tolist(), \
                        f"mode {mode} row {r} threads {threads} table {pg is not None}"
        # a row subset gives the same lines as the full call
        sub = [7, 2, 2, 10]
        full = orc.topk(L, lens, k, mode, width=width, pages=pages, page_size=P)
        part = orc.topk(L, lens, k, mode, width=width, pages=pages, page_size=P, rows=sub,
                        threads=2)
        assert part.tolist() == full[sub].tolist(), f"mode {mode}: rows= subset"
        # ordered results, row by row against the rank definition
        for threads in (1, 4):
            out, ids, valid = orc.topk_ordered(L, lens, k, mode, width=width, pages=pages,
                                               page_size=P, threads=threads)
            for r in range(rows):
                keys = orc.row_keys(L[r, :width], int(lens[r]), mode)
                sel = _ordered_by_rank(keys, keys.size, k)
                want_ids = sel + [-1] * (k - len(sel))
                want_out = []
                for i in want_ids:
                    o = i
                    if i >= 0 and mode == BLOCK and keys[i] == 0x007F:
                        o = -1
                    if o >= 0:
                        o = int(pages[r, o // P]) * P + o % P
                    want_out.append(o)
                ctx = f"ordered mode {mode} row {r} threads {threads}"
                assert int(valid[r]) == len(sel), ctx
                assert ids[r].tolist() == want_ids, ctx
                assert out[r].tolist() == want_out, ctx


def pin_vector_maxima(orc):
    """The side array of vector maxima (vLLM kimi_k3 indexer page,
    IndexerScore epilogue): closed forms on monotone rows (the maximum of a
    vector is its last valid logit when values rise, its first when they
    fall), nothing past the valid length, zero for vectors holding no valid
    logit, and on random rows every entry is attained by a valid logit of its
    vector and dominates the others."""
    width = 100
    rise = (0x3F80 + np.arange(width)).astype(np.uint16)       # 1.0 and up
    fall = rise[::-1].copy()
    for v in (0, 1, 7, 8, 9, 93, 100):
        t = orc.vector_maxima(rise[None, :], [v], width)[0]
        assert t.shape == (13,)
        for j in range(13):
            lastv = min(8 * j + 8, v) - 1
            want = int(orc.key(rise[lastv])) if lastv >= 8 * j else 0
            assert int(t[j]) == want, (v, j)
        t = orc.vector_maxima(fall[None, :], [v], width)[0]
        for j in range(13):
            want = int(orc.key(fall[8 * j])) if 8 * j < v else 0
            assert int(t[j]) == want, (v, j)
    # the largest value sits past the length: it must not show
    row = np.full(16, 0x3F80, np.uint16)
    row[12] = 0x7F80                                           # +inf past v = 12
    t = orc.vector_maxima(row[None, :], [12], 16)[0]
    assert t.tolist() == [int(orc.key(0x3F80))] * 2
    # negative NaNs only: key 0; a positive NaN: above +inf
    t = orc.vector_maxima(np.array([[0xFFFF] * 8 + [0x7FC1] + [0] * 7], np.uint16), [16], 16)[0]
    assert int(t[0]) == 0 and int(t[1]) > int(orc.key(0x7F80))
    rng = np.random.Generator(np.random.PCG64(4242))
    for trial in range(20):
        width = int(rng.integers(1, 300))
        rows = 3
        L = rng.integers(0, 1 << 16, size=(rows, width), dtype=np.uint32).astype(np.uint16)
        vl = rng.integers(-3, width + 4, size=rows)
        t = orc.vector_maxima(L, vl, width)
        for r in range(rows):
            v = max(0, min(int(vl[r]), width))
            keys = orc.key(L[r])
            for j in range((width + 7) // 8):
                seg = keys[8 * j:min(8 * j + 8, v)]
                if seg.size == 0:
                    assert int(t[r, j]) == 0
                else:
                    assert int(t[r, j]) in set(int(x) for x in seg)
                    assert all(int(t[r, j]) >= int(x) for x in seg)


def pin_vector_maxima_bound(orc):
    """The property the select relies on: the k-th largest vector maximum is
    at most the row's k-th largest key, and at least k keys lie at or above
    it."""
    rng = np.random.Generator(np.random.PCG64(4243))
    for trial in range(12):
        k = int(rng.integers(1, 40))
        width = int(rng.integers(16 * k, 16 * k + 200))
        row = rng.integers(0, 1 << 16, size=width, dtype=np.uint32).astype(np.uint16)
        if trial % 2:
            row = (rng.standard_normal(width, dtype=np.float32).view(np.uint32) >> 16).astype(
                np.uint16)  # normal values, truncated to BF16
        t = orc.vector_maxima(row[None, :], [width], width)[0]
        low = int(np.sort(t)[::-1][k - 1])
        keys = orc.row_keys(row, width, 0)
        T = orc.threshold(keys, k)[0]
        assert low <= int(T)
        assert int((keys >= low).sum()) >= k


ALL_PINS = [
    pin_key_fixed_points,
    pin_key_bijection,
    pin_key_follows_float_order,
    pin_key_nan_placement,
    pin_is_nan,
    pin_block_key_max,
    pin_block_key_nan,
    pin_block_key_special,
    pin_row_keys_block,
    pin_bruteforce_tiny_rows,
    pin_threshold_by_numpy_sort,
    pin_values_match_numpy_topk,
    pin_short_rows,
    pin_clamped_lengths,
    pin_constant_row,
    pin_block_neg_inf_rows,
    pin_poison_not_selected,
    pin_page_transform_roundtrip,
    pin_worked_examples,
    pin_ordered_rank_definition,
    pin_ordered_worked_cases,
    pin_multirow_driver,
    pin_vector_maxima,
    pin_vector_maxima_bound,
]


def failing_pins(orc):
    """Names of the pins this oracle fails (crashes count as failures)."""
    bad = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001
            bad.append(f"{pin.__name__}: {type(e).__name__}: {e}"[:200])
    return bad


if __name__ == "__main__":
    # python oracle_pins.py <library>: run every pin against one compiled copy
    # of the oracle; exit status 0 when all pass, 1 when any fails.
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import oracle as _oracle

    failures = failing_pins(_oracle.Oracle(sys.argv[1]))
    for line in failures:
        print(line)
    sys.exit(1 if failures else 0)
