"""GPU parity of the ordered results (topk_bf16_rows_ordered) against the
oracle's ordered definition, element by element: out, ids and valid must be
bit-identical (the result is unique: ascending indices, ties at the k-th key
from the lowest indices).  Every selection path is driven: sampled, tie pass,
misjudged and overflowing samples, forced direct, short rows; one-workgroup
rows and team rows; both modes; with and without a block table."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from checker import check
from test_parity_gpu import (EDGE, MULTI_BATCH, PAGE_CASES, _make, _sampled_positions_wg,
                             _sampled_vectors_team, with_pages)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

T = None


def setup_module(module):
    global T
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_wise_amd as _T
    T = _T
    T.library()


def run_ordered(d, force_direct=False, want_ids=True):
    L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
    VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
    P = None if d.get("pages") is None else torch.from_numpy(np.ascontiguousarray(d["pages"])).cuda()
    rows = L.shape[0]
    pc = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    out, valid, ids = T.topk_bf16_rows_ordered(L, VL, d["k"], d["mode"], block_table=P,
                                               page_size=d.get("page_size") or 64,
                                               width=d["width"], want_ids=want_ids,
                                               force_direct=force_direct, path_codes=pc)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), valid.cpu().numpy(),
            None if ids is None else ids.cpu().numpy(), pc.cpu().numpy())


def oracle_ordered(d, rows=None):
    L, vl, P = d["logits"], d["valid_len"], d.get("pages")
    if rows is not None:
        L, vl = L[rows], np.asarray(vl)[rows]
        P = None if P is None else P[rows]
    return oracle.topk_ordered(L, vl, d["k"], d["mode"], width=d["width"], pages=P,
                               page_size=d.get("page_size") or 64, threads=16)


def assert_ordered(g, o, rows=None, ctx=""):
    out, valid, ids = g[0], g[1], g[2]
    if rows is not None:
        out, valid = out[rows], valid[rows]
        ids = None if ids is None else ids[rows]
    oo, oi, ov = o
    bad = np.nonzero(valid != ov)[0]
    assert bad.size == 0, f"{ctx} valid differs in rows {bad[:8]}: {valid[bad[:8]]} vs {ov[bad[:8]]}"
    for name, a, b in (("out", out, oo), ("ids", ids, oi)):
        if a is None:
            continue
        rb = np.nonzero((a != b).any(axis=1))[0]
        if rb.size:
            r = rb[0]
            j = np.nonzero(a[r] != b[r])[0][:6]
            raise AssertionError(f"{ctx} {name} differs in {rb.size} rows, first row {r} at "
                                 f"{j}: gpu {a[r][j]} oracle {b[r][j]}")


def _paths(pc):
    u, c = np.unique(pc, return_counts=True)
    return dict(zip(u.tolist(), c.tolist()))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_ordered_workloads(cfg):
    d = W.make(cfg)
    rows = d["logits"].shape[0]
    print(f"ordered workload {cfg} {d['name']} rows={rows}", flush=True)
    g = run_ordered(d)
    # the oracle on every row up to 512 rows; beyond, on every 16th row and
    # on every special row of the edge workload (r % 10 == 9: constant, all
    # -inf, NaN, signed-zero and random-bit rows)
    sel = None if rows <= 512 else np.union1d(np.arange(0, rows, 16), np.arange(9, rows, 10))
    assert_ordered(g, oracle_ordered(d, sel), sel, ctx=d["name"])
    paths = _paths(g[3])
    print("paths", paths, flush=True)
    assert -9 not in paths


@pytest.mark.parametrize("width,k,mode,kind,pad", EDGE)
def test_ordered_edge_shapes(width, k, mode, kind, pad):
    rng = np.random.Generator(np.random.PCG64(width * 7 + k + 13 * mode))
    lens = [width, width - 1, max(0, width // 3), -5, width + 100, k]
    d = _make(rng, 6, width, k, mode, kind, stride_pad=pad, lens=lens, pages=(width % 2 == 0))
    print(f"ordered edge width={width} k={k} mode={mode} kind={kind}", flush=True)
    o = oracle_ordered(d)
    for fd in (False, True):
        assert_ordered(run_ordered(d, force_direct=fd), o, ctx=f"force_direct={fd}")


def test_ordered_without_ids():
    rng = np.random.Generator(np.random.PCG64(5))
    for width, mode in ((16384, 0), (150000, 0), (40000, 1)):
        d = _make(rng, 4, width, 512, mode, "ties", pages=True)
        g = run_ordered(d, want_ids=False)
        assert g[2] is None
        assert_ordered(g, oracle_ordered(d), ctx=f"width={width}")


def _row(L, k, mode=0):
    rows, width = L.shape
    return dict(logits=L, valid_len=np.full(rows, width, np.int32), k=k, mode=mode,
                width=width, pages=None, page_size=0)


def _crafted():
    """Rows that drive each selection path (built as in the unordered path
    tests), with the path they must take."""
    cases = []
    width = 16384
    L = np.full((2, width), 0x3F00, np.uint16)
    pos = _sampled_positions_wg(width // 8)
    L[:, pos] = (0x4000 + np.arange(pos.size) % 0x700).astype(np.uint16)
    cases.append(("wg misjudged", _row(L, 512), "PATH_DIRECT_MISJUDGED"))
    rng = np.random.Generator(np.random.PCG64(79))
    L = W.f32_to_bf16_bits(np.abs(rng.standard_normal((2, width), dtype=np.float32)) + 1)
    L[:, pos] = 0x3C00
    cases.append(("wg overflow", _row(L, 512), "PATH_DIRECT_OVERFLOW"))
    # one workgroup, the k-th key is the cutoff and it is tied: the tie pass
    L = np.full((2, width), 0x3F00, np.uint16)
    L[:, ::4] = 0x3F80
    L[:, pos[:5]] = (0x4000 + np.arange(5)).astype(np.uint16)
    cases.append(("wg ties", _row(L, 512), None))
    width = 150000
    L = np.full((2, width), 0x3F80, np.uint16)
    tpos = (_sampled_vectors_team(width // 8) * 8)[:20]
    L[:, tpos] = (0x4000 + np.arange(20)).astype(np.uint16)
    cases.append(("team skipped ties", _row(L, 512), "PATH_DIRECT_MISJUDGED"))
    width = 40000
    L = np.full((2, width), 0x3F00, np.uint16)
    L[:, ::4] = 0x3F80
    L[:, (_sampled_vectors_team(width // 8) * 8 + 1)[:5]] = (0x4000 + np.arange(5)).astype(np.uint16)
    cases.append(("team ties collected", _row(L, 512), "PATH_SAMPLED_TIES"))
    width = 150000
    L = np.full((2, width), 0x3F00, np.uint16)
    L[:, ::64] = 0x3F80
    L[:, (_sampled_vectors_team(width // 8) * 8 + 1)[:5]] = (0x4000 + np.arange(5)).astype(np.uint16)
    cases.append(("team cutoff below ties", _row(L, 512), "PATH_SAMPLED"))
    rng = np.random.Generator(np.random.PCG64(4500))
    L = W.f32_to_bf16_bits(rng.standard_normal((2, 36000), dtype=np.float32))
    cases.append(("team member overflow", _row(L, 2048, mode=1), "PATH_DIRECT_OVERFLOW"))
    return cases


@pytest.mark.parametrize("case", range(7))
def test_ordered_crafted_paths(case):
    name, d, path = _crafted()[case]
    print(f"ordered crafted {name}", flush=True)
    g = run_ordered(d)
    assert_ordered(g, oracle_ordered(d), ctx=name)
    if path is not None:
        assert np.all(g[3] == getattr(T, path)), (name, g[3])


def test_ordered_then_unordered_share_scratch():
    """Ordered and unordered calls of team rows alternate on one stream: each
    stays exact (the ordered call's records live after the team slices)."""
    rng = np.random.Generator(np.random.PCG64(77))
    d1 = _make(rng, 24, 150000, 512, 0, "normal")
    d2 = _make(rng, 40, 70000, 2048, 1, "bits")
    for d in (d1, d2, d1):
        assert_ordered(run_ordered(d), oracle_ordered(d))
        L = torch.from_numpy(d["logits"].view(np.int16)).cuda()
        VL = torch.from_numpy(d["valid_len"]).cuda()
        out = T.topk_bf16_rows(L, VL, d["k"], d["mode"], width=d["width"])
        torch.cuda.synchronize()
        want = oracle.topk(d["logits"], d["valid_len"], d["k"], d["mode"], width=d["width"],
                           threads=16)
        bad = check(oracle.default(), d, out.cpu().numpy(), want)
        assert not bad, "\n".join(bad)


def test_ordered_graph_replays():
    """Ordered calls captured in one HIP graph (a one-workgroup row batch
    with a block table, a token team, a block team) and replayed several
    times, with an eager ordered call and synchronizations between the
    replays: every replay's out, ids and valid equal the oracle's (no memset
    is recorded, and the order records and counts in the team scratch are
    rewritten by every call)."""
    ds = [W.make(2, rows=48, width=16384, seed=501), W.make(3, rows=5, width=60000, seed=502),
          W.make(4, rows=6, width=150000, seed=503)]
    # eager work in between, on the same stream and scratch
    other = W.make(3, rows=7, width=50000, seed=504)
    refs = [oracle_ordered(d) for d in ds]
    s = torch.cuda.Stream()
    dev = []
    for d in ds:
        L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
        VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
        P = None if d.get("pages") is None else torch.from_numpy(d["pages"]).cuda()
        dev.append((L, VL, P))

    def calls():
        return [T.topk_bf16_rows_ordered(L, VL, d["k"], d["mode"], block_table=P,
                                         page_size=d.get("page_size") or 64, width=d["width"])
                for d, (L, VL, P) in zip(ds, dev)]

    # the stream's scratch sized for every shape before the first call and
    # the capture: calls never replace a reserved (or captured) scratch
    for d in ds + [other]:
        T.reserve_scratch(d["logits"].shape[0], d["width"], d["k"], d["mode"], stream=s)
    with torch.cuda.stream(s):
        calls()  # first use on this stream: the scratch is set up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = calls()
    for rep in range(3):
        with torch.cuda.stream(s):
            for trio in outs:
                for t in trio:
                    t.fill_(-7)
            L = torch.from_numpy(other["logits"].view(np.int16)).cuda()
            VL = torch.from_numpy(other["valid_len"]).cuda()
            go = T.topk_bf16_rows_ordered(L, VL, other["k"], other["mode"], width=other["width"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"ordered graph replay {rep}", flush=True)
        for d, (o, v, i), ref in zip(ds, outs, refs):
            assert_ordered((o.cpu().numpy(), v.cpu().numpy(), i.cpu().numpy()), ref,
                           ctx=f"replay {rep} {d['name']}")
        assert_ordered(tuple(t.cpu().numpy() for t in go), oracle_ordered(other), ctx="eager")


@pytest.mark.parametrize("rows,width,k,mode,kind", MULTI_BATCH)
def test_ordered_team_multi_batch(rows, width, k, mode, kind):
    """Ordered results of launches with more rows than one team batch holds
    (the later batches' records, counts, ids and outputs start at row0 > 0)."""
    rng = np.random.Generator(np.random.PCG64(rows + width + 1))
    lens = rng.integers(k + 1, width + 1, size=rows).astype(np.int32)
    lens[::7] = width
    lens[3::50] = k // 2
    d = _make(rng, rows, width, k, mode, kind, lens=lens)
    print(f"ordered multi-batch rows={rows} width={width}", flush=True)
    assert_ordered(run_ordered(d), oracle_ordered(d), ctx=f"rows={rows} width={width}")


@pytest.mark.parametrize("P,width,mode", PAGE_CASES)
def test_ordered_page_sizes(P, width, mode):
    rng = np.random.Generator(np.random.PCG64(P * 31 + width + mode + 1))
    k = 512 if mode == 0 else 1024
    lens = [width, width - 5, width // 2, k - 3, 3 * k]
    d = with_pages(_make(rng, 5, width, k, mode, "normal", lens=lens), P, rng)
    print(f"ordered page size {P} width {width} mode {mode}", flush=True)
    o = oracle_ordered(d)
    for fd in (False, True):
        assert_ordered(run_ordered(d, force_direct=fd), o, ctx=f"P={P} force_direct={fd}")
