"""GPU parity of the vector-max bound (topk_bf16_rows_tops) and of the
library's side array of vector maxima (topk_bf16_vector_maxima), through
the C ABI, against the CPU oracle.

The side array the selection reads comes from the oracle's definition
(oracle_vector_maxima), so a selection test does not depend on the
library's own maxima kernel; that kernel is checked against the same
definition separately, and once end to end."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from checker import check

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


def _tops_host(d, pad=0):
    """The oracle's maxima in a [rows, tops_stride] array (stride a multiple
    of 8, `pad` words of 8 more)."""
    width = d["width"]
    t = oracle.vector_maxima(d["logits"][:, :width], d["valid_len"], width)
    nv = (width + 7) // 8
    stride = max(8, -(-nv // 8) * 8) + 8 * pad
    out = np.full((t.shape[0], stride), 0xBEEF, np.uint16)  # never read past nv
    out[:, :nv] = t
    return out


def _dev(d):
    L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
    VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
    P = None if d.get("pages") is None else torch.from_numpy(np.ascontiguousarray(d["pages"])).cuda()
    return L, VL, P


def run_tops(d, tops=None, force_direct=False, pad=0):
    L, VL, P = _dev(d)
    if tops is None:
        tops = torch.from_numpy(_tops_host(d, pad).view(np.int16)).cuda()
    rows = L.shape[0]
    pc = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    out = T.topk_bf16_rows_tops(L, VL, d["k"], tops, d["mode"], block_table=P,
                                page_size=d.get("page_size") or 64, width=d["width"],
                                force_direct=force_direct, path_codes=pc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), pc.cpu().numpy()


def run_oracle(d):
    return oracle.topk(d["logits"], d["valid_len"], d["k"], d["mode"], width=d["width"],
                       pages=d.get("pages"), page_size=d.get("page_size") or 64, threads=16)


def assert_parity(d, g, o):
    bad = check(oracle.default(), d, g, o)
    assert not bad, "\n".join(bad)


def _paths(pc):
    u, c = np.unique(pc, return_counts=True)
    return dict(zip(u.tolist(), c.tolist()))


def test_vector_maxima_match_the_definition():
    rng = np.random.Generator(np.random.PCG64(515))
    for width in (1, 7, 8, 9, 63, 64, 65, 1000, 16384, 16391, 150000):
        rows = 5
        stride = (width + 7) // 8 * 8
        L = np.full((rows, stride), W.POISON, np.uint16)
        L[:, :width] = rng.integers(0, 1 << 16, size=(rows, width), dtype=np.uint32).astype(
            np.uint16)
        vl = np.array([width, 0, max(0, width - 3), -4, width + 11], np.int32)
        d = dict(logits=L, valid_len=vl, width=width)
        want = oracle.vector_maxima(L[:, :width], vl, width)
        Ld, VL, _ = _dev(d)
        got = T.vector_maxima(Ld, VL, width=width)
        torch.cuda.synchronize()
        got = got.cpu().numpy().view(np.uint16)
        nv = (width + 7) // 8
        assert np.array_equal(got[:, :nv], want), f"width {width}"
        assert not got[:, nv:-(-nv // 8) * 8].any(), f"width {width}: padding"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(cfg):
    d = W.make(cfg)
    print(f"tops workload {cfg} {d['name']} rows={d['logits'].shape[0]}", flush=True)
    g, pc = run_tops(d)
    assert_parity(d, g, run_oracle(d))
    paths = _paths(pc)
    print("paths", paths, flush=True)
    assert -9 not in paths
    if cfg in (1, 3):
        assert paths == {T.PATH_TOPS: d["logits"].shape[0]}, paths
    if cfg == 2:
        nvec = (np.minimum(np.maximum(d["valid_len"], 0), d["width"]) + 7) // 8
        on_bound = nvec >= 2 * d["k"]
        assert np.all(pc[on_bound] == T.PATH_TOPS), _paths(pc[on_bound])
    if cfg in (4, 5):  # block mode, and rows of fewer than 2k vectors: no bound
        assert T.PATH_TOPS not in paths


def test_maxima_from_the_library_end_to_end():
    d = W.make(2, rows=96, seed=516)
    L, VL, P = _dev(d)
    tops = T.vector_maxima(L, VL, width=d["width"])
    g, pc = run_tops(d, tops=tops)
    assert_parity(d, g, run_oracle(d))


def _rows(rng, rows, width, kind):
    if kind == "normal":
        return W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32))
    if kind == "bits":
        return rng.integers(0, 1 << 16, size=(rows, width), dtype=np.uint32).astype(np.uint16)
    if kind == "crowded":
        lv = W.f32_to_bf16_bits(rng.standard_normal(200).astype(np.float32) * 2.0)
        w = 1.0 / np.arange(1, 201)
        return lv[rng.choice(200, size=(rows, width), p=w / w.sum())]
    if kind == "negative":
        return W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32) - 8.0)
    raise ValueError(kind)


def _make(rng, rows, width, k, kind, lens=None, pages=None, pad=0):
    stride = (width + 7) // 8 * 8 + 8 * pad
    L = np.full((rows, stride), W.POISON, np.uint16)
    L[:, :width] = _rows(rng, rows, width, kind)
    lens = np.full(rows, width, np.int32) if lens is None else np.asarray(lens, np.int32)
    for r in range(rows):
        L[r, max(0, min(int(lens[r]), width)):] = W.POISON
    P, psz = None, 0
    if pages:
        psz = pages
        npg = (width + psz - 1) // psz
        P = np.stack([rng.permutation(npg) for _ in range(rows)]).astype(np.int32)
    return dict(logits=L, valid_len=lens, k=k, mode=0, width=width, pages=P, page_size=psz)


SHAPES = [
    # width, k, kind, pages: one word of maxima per thread, then 2, 4 and 8
    (16384, 512, "normal", 64), (16384, 1, "bits", 0), (16384, 64, "crowded", 16),
    (10000, 512, "negative", 0), (20000, 1024, "normal", 0), (40000, 512, "crowded", 64),
    (70001, 2048, "bits", 0), (150000, 512, "crowded", 0), (262144, 2048, "normal", 0),
]


@pytest.mark.parametrize("width,k,kind,pages", SHAPES)
def test_shapes(width, k, kind, pages):
    """Ragged lengths (partial last vectors, n <= k rows, rows with fewer
    than 2k vectors on either side of 16384 logits, lengths out of range),
    block tables, padded strides, on the bound and on the forced direct
    path."""
    rng = np.random.Generator(np.random.PCG64(width + 7 * k))
    lens = [width, width - 1, width - 7, k, k + 1, 16 * k + 3, min(width, 16384) - 5,
            min(width, 24000) - 9, -2, width + 5]
    rows = len(lens)
    d = _make(rng, rows, width, k, kind, lens=lens, pages=pages or None, pad=1)
    print(f"tops shape width={width} k={k} kind={kind} pages={pages}", flush=True)
    o = run_oracle(d)
    g, pc = run_tops(d, pad=2)
    assert_parity(d, g, o)
    v = np.minimum(np.maximum(np.array(lens), 0), width)
    nvec = (v + 7) // 8
    for r in range(rows):
        if v[r] <= k:
            assert pc[r] == T.PATH_SHORT, (r, pc[r])
        elif nvec[r] < 2 * k:
            want = {T.PATH_SAMPLED, T.PATH_SAMPLED_TIES, T.PATH_DIRECT_MISJUDGED,
                    T.PATH_DIRECT_OVERFLOW} if v[r] <= 16384 else {T.PATH_DIRECT_DENSE}
            assert pc[r] in want, (r, pc[r])
        elif (width + 7) // 8 >= 2 * k:
            assert pc[r] in (T.PATH_TOPS, T.PATH_DIRECT_OVERFLOW), (r, pc[r])
    g, pc = run_tops(d, force_direct=True)
    assert_parity(d, g, o)


def test_fallbacks_on_the_bound():
    """Rows the bound cannot serve: a constant row (every vector hot: the
    hot lists overflow), a row of negative NaNs only (every key 0, so the
    bound is 0), and a row whose maxima are tied across most vectors."""
    width, k = 16384, 256
    rows = 4
    L = np.full((rows, width), 0x3F80, np.uint16)                 # constant 1.0
    L[1] = 0xFFFF                                                  # keys 0
    rng = np.random.Generator(np.random.PCG64(517))
    L[2] = np.where(rng.random(width) < 0.2, 0x4000, 0x3F00).astype(np.uint16)
    L[3] = W.f32_to_bf16_bits(rng.standard_normal(width, dtype=np.float32))
    d = dict(logits=L, valid_len=np.full(rows, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_tops(d)
    assert_parity(d, g, run_oracle(d))
    assert pc[0] == T.PATH_DIRECT_OVERFLOW, pc
    assert pc[1] == T.PATH_DIRECT_MISJUDGED, pc
    assert pc[2] == T.PATH_DIRECT_OVERFLOW, pc
    assert pc[3] == T.PATH_TOPS, pc


def test_many_rows_throughput_variant():
    """More rows than resident workgroups (the throughput variant)."""
    d = W.make(2, rows=3000, seed=518)
    g, pc = run_tops(d)
    assert_parity(d, g, run_oracle(d))
