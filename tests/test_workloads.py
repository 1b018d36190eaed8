"""The seeded generators produce the shapes and value mixes stated for each
workload (no selection arithmetic here)."""
import numpy as np

import workloads as W


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_deterministic():
    a = W.make(2, rows=16, width=1024)
    b = W.make(2, rows=16, width=1024)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["valid_len"], b["valid_len"])


def test_shapes_and_poison():
    for cfg, rows, width in ((1, 4, 1000), (2, 20, 4096), (3, 3, 15000), (4, 3, 40000),
                             (5, 40, 4096)):
        d = W.make(cfg, rows=rows, width=width)
        L = d["logits"]
        assert L.shape == (rows, (width + 7) // 8 * 8) and L.dtype == np.uint16
        assert d["row_stride"] % 8 == 0
        for r in range(rows):
            v = int(d["valid_len"][r])
            assert 0 <= v <= width
            assert np.all(L[r, v:] == W.POISON)


def test_ragged_and_pages():
    d = W.make(2, rows=100, width=4096)
    vl = d["valid_len"]
    assert (vl <= d["k"]).sum() == 10
    assert (vl > d["k"]).sum() == 90
    P = d["pages"]
    assert P.shape == (100, 4096 // 64)
    for r in range(100):
        assert np.array_equal(np.sort(P[r]), np.arange(64))


def test_crowded_levels():
    d = W.make(3, rows=2, width=20000)
    assert len(np.unique(d["logits"][:, :20000])) <= 200
    assert len(np.unique(d["logits"][:, :20000])) > 100


def test_block_rows():
    d = W.make(4, rows=4, width=65536)
    assert np.all(d["valid_len"] % 8 == 0) and np.all(d["valid_len"] >= 16384)
    L = d["logits"][:, :65536].reshape(4, -1, 8)
    allinf = np.all(L == W.BF16_NEG_INF, axis=2)
    assert 0.005 < allinf.mean() < 0.02


def test_edge_rows():
    d = W.make(5, rows=80, width=4096)
    L = d["logits"]
    kinds = {((r // 10) % 8): r for r in range(9, 80, 10)}
    assert len(np.unique(L[kinds[0]])) == 1
    assert np.all(L[kinds[1]] == W.BF16_NEG_INF)
    assert np.isnan(_f(L[kinds[2]])).sum() == 3000
    z = L[kinds[3]]
    assert ((z == 0) | (z == 0x8000)).sum() == 4096 - 2047
    assert (z == 0x8000).any() and (z == 0).any()
    spec = W._special_patterns()
    assert all(np.isin(spec, L[kinds[4]]))
