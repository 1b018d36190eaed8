"""GPU parity: libtopk (through its C ABI) against the CPU oracle.

Every workload runs at full size with every row checked, plus reduced and
edge-case shapes; the direct radix path is exercised both on request and on
rows built to defeat the sampled cutoff.
"""
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


def _dev(d):
    L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
    VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
    P = None if d.get("pages") is None else torch.from_numpy(np.ascontiguousarray(d["pages"])).cuda()
    return L, VL, P


def run_gpu(d, force_direct=False, stream=None):
    L, VL, P = _dev(d)
    rows = L.shape[0]
    pc = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    out = T.topk_bf16_rows(L, VL, d["k"], d["mode"], block_table=P,
                           page_size=d.get("page_size") or 64, width=d["width"],
                           force_direct=force_direct, path_codes=pc, stream=stream)
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


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(cfg):
    d = W.make(cfg)
    print(f"workload {cfg} {d['name']} rows={d['logits'].shape[0]}", flush=True)
    g, pc = run_gpu(d)
    o = run_oracle(d)
    assert_parity(d, g, o)
    paths = _paths(pc)
    print("paths", paths, flush=True)
    assert -9 not in paths
    fallback = paths.get(T.PATH_DIRECT_MISJUDGED, 0) + paths.get(T.PATH_DIRECT_OVERFLOW, 0)
    assert fallback <= max(1, d["logits"].shape[0] // 100), paths


@pytest.mark.parametrize("cfg,rows,width", [(1, 4, 16384), (2, 64, 16384), (3, 8, 150000),
                                            (4, 6, 1048576), (5, 160, 16384)])
def test_workload_direct_path(cfg, rows, width):
    d = W.make(cfg, rows=rows, width=width, seed=100 + cfg)
    g, pc = run_gpu(d, force_direct=True)
    assert_parity(d, g, run_oracle(d))
    n = np.minimum(np.maximum(d["valid_len"], 0), width)
    if d["mode"] == 1:
        n = (n + 7) // 8
    long_rows = n > d["k"]
    assert np.all(pc[long_rows] == T.PATH_DIRECT_FORCED)
    assert np.all(pc[~long_rows] == T.PATH_SHORT)


def _random_rows(rng, rows, width, kind):
    if kind == "normal":
        x = rng.standard_normal((rows, width), dtype=np.float32)
        return W.f32_to_bf16_bits(x)
    if kind == "bits":
        return rng.integers(0, 1 << 16, size=(rows, width), dtype=np.uint32).astype(np.uint16)
    if kind == "ties":
        lv = np.array([0x3F80, 0x4000, 0xBF80, 0x0000, 0x8000, 0xFF80, 0x7F80], np.uint16)
        return lv[rng.integers(0, lv.size, size=(rows, width))]
    if kind == "negative":  # every value below zero: the cutoff is negative
        x = rng.standard_normal((rows, width), dtype=np.float32) - 8.0
        return W.f32_to_bf16_bits(x)
    if kind in ("neg_ties", "crowded"):
        # a few levels with Zipf weights: the cutoff falls on a heavily tied
        # key (negative levels, or N(0, 2) levels)
        nlv = 30 if kind == "neg_ties" else 200
        lvf = rng.standard_normal(nlv).astype(np.float32) * 2.0
        if kind == "neg_ties":
            lvf = -np.abs(lvf) - 0.5
        lv = W.f32_to_bf16_bits(lvf)
        w = 1.0 / np.arange(1, nlv + 1)
        return lv[rng.choice(nlv, size=(rows, width), p=w / w.sum())]
    raise ValueError(kind)


def _make(rng, rows, width, k, mode, kind, stride_pad=0, lens=None, pages=False):
    stride = (width + 7) // 8 * 8 + 8 * stride_pad
    L = np.full((rows, stride), W.POISON, np.uint16)
    L[:, :width] = _random_rows(rng, rows, width, kind)
    if lens is None:
        lens = np.full(rows, width, np.int32)
    lens = np.asarray(lens, np.int32)
    for r in range(rows):
        v = max(0, min(int(lens[r]), width))
        L[r, v:] = W.POISON
    P = None
    if pages:
        npg = (width + 63) // 64
        P = np.stack([rng.permutation(npg) for _ in range(rows)]).astype(np.int32)
    return dict(logits=L, valid_len=lens, k=k, mode=mode, width=width, pages=P,
                page_size=64 if pages else 0, name="edge")


EDGE = [
    # (width, k, mode, kind, stride_pad)
    (1, 1, 0, "bits", 0), (7, 3, 0, "bits", 1), (9, 8, 0, "normal", 0), (100, 1, 0, "ties", 0),
    (1000, 999, 0, "bits", 0), (2049, 2048, 0, "normal", 0), (5000, 17, 0, "ties", 2),
    (16384, 2048, 0, "bits", 0), (16385, 512, 0, "normal", 0), (16392, 100, 0, "ties", 0),
    (40000, 1, 0, "normal", 0), (70001, 2048, 0, "bits", 3),
    (8, 1, 1, "bits", 0), (17, 2, 1, "bits", 0), (800, 50, 1, "ties", 0),
    (32768, 2048, 1, "normal", 0), (32776, 1024, 1, "bits", 0), (100001, 7, 1, "normal", 1),
    (300000, 2048, 1, "ties", 0),
    # negative cutoffs and heavily tied cutoffs, one workgroup and team rows
    (16384, 512, 0, "neg_ties", 0), (8000, 300, 1, "neg_ties", 0), (12000, 300, 0, "negative", 0),
    (60000, 512, 0, "negative", 0), (60000, 512, 0, "neg_ties", 1), (40000, 100, 0, "neg_ties", 0),
    (150000, 1024, 0, "crowded", 0), (200000, 2048, 1, "neg_ties", 0), (33000, 2048, 1, "negative", 0),
]


@pytest.mark.parametrize("width,k,mode,kind,pad", EDGE)
def test_edge_shapes(width, k, mode, kind, pad):
    rng = np.random.Generator(np.random.PCG64(width * 7 + k + 13 * mode))
    rows = 6
    lens = [width, width - 1, max(0, width // 3), -5, width + 100, k]
    d = _make(rng, rows, width, k, mode, kind, stride_pad=pad, lens=lens, pages=(width % 2 == 0))
    print(f"edge width={width} k={k} mode={mode} kind={kind}", flush=True)
    for fd in (False, True):
        g, pc = run_gpu(d, force_direct=fd)
        assert_parity(d, g, run_oracle(d))


def test_block_mode_specials():
    """NaN blocks (either sign) above the pinned block, -inf blocks as -1,
    +0/-0 blocks, partial newest block."""
    rng = np.random.Generator(np.random.PCG64(77))
    width, k = 8 * 6000, 600
    rows = 4
    L = W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32))
    B = L.reshape(rows, -1, 8)
    nb = B.shape[1]
    B[0, rng.choice(nb, 300, replace=False), 3] = 0xFFC0      # -NaN in 300 blocks
    B[1, rng.choice(nb, 700, replace=False), :] = 0xFF80      # 700 -inf blocks
    B[2, :, :] = 0xFF80                                        # all -inf
    B[2, rng.choice(nb, 100, replace=False), 5] = 0x8000      # some -0 blocks
    B[3, :, :] = 0x8000
    B[3, rng.choice(nb, 50, replace=False), 0] = 0x0000        # +0 beats -0
    d = dict(logits=L, valid_len=np.array([width, width - 3, width, 8 * 700 + 5], np.int32),
             k=k, mode=1, width=width, pages=None, page_size=0)
    for fd in (False, True):
        g, pc = run_gpu(d, force_direct=fd)
        assert_parity(d, g, run_oracle(d))


def test_block_mode_page_transform():
    rng = np.random.Generator(np.random.PCG64(78))
    d = _make(rng, 5, 8 * 4000, 300, 1, "normal", lens=[32000, 31999, 100, 2400, 8 * 300],
              pages=True)
    g, _ = run_gpu(d)
    assert_parity(d, g, run_oracle(d))


def _sampled_positions_wg(nvec):
    """Positions the one-workgroup token kernel samples: logit (vid // 512)
    mod 8 of vector vid, at either workgroup size (with 512 threads, logit
    j mod 8 of the vector staged in slot j)."""
    vid = np.arange(nvec)
    return vid * 8 + (vid // 512) % 8


# 2 rows: 1024-thread workgroups (no more rows than compute units); 300 rows:
# 512-thread workgroups, all resident
CRAFTED_ROWS = [2, 300]


@pytest.mark.parametrize("rows", CRAFTED_ROWS)
def test_crafted_misjudged_row_takes_direct_path(rows):
    """Sampled positions hold the row's largest values and everything else is
    lower, so fewer than k keys lie at or above the cutoff."""
    width, k = 16384, 512
    L = np.full((rows, width), 0x3F00, np.uint16)             # 0.5 everywhere
    pos = _sampled_positions_wg(width // 8)
    L[:, pos] = (0x4000 + np.arange(pos.size) % 0x700).astype(np.uint16)
    d = dict(logits=L, valid_len=np.full(rows, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_DIRECT_MISJUDGED), pc


@pytest.mark.parametrize("rows", CRAFTED_ROWS)
def test_crafted_overflow_row_takes_direct_path(rows):
    """Sampled positions hold the smallest values, so almost every other key
    lies above the cutoff and the survivor regions overflow."""
    rng = np.random.Generator(np.random.PCG64(79))
    width, k = 16384, 512
    L = W.f32_to_bf16_bits(np.abs(rng.standard_normal((rows, width), dtype=np.float32)) + 1)
    pos = _sampled_positions_wg(width // 8)
    L[:, pos] = 0x3C00                                         # tiny positives
    d = dict(logits=L, valid_len=np.full(rows, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_DIRECT_OVERFLOW), pc


@pytest.mark.parametrize("rows", [2600, 2605])
def test_many_rows_mixed(rows):
    """More token rows than workgroups resident at once (the throughput
    kernel, whose workgroups take the rows of each group of 8 in a hashed
    rotation; 2605 rows leave a last group of 5): every kind of row next to
    every other in one launch, ragged and short lengths, rows built to take
    each fallback, and the last rows of the launch; on the sampled path and
    the forced direct path."""
    rng = np.random.Generator(np.random.PCG64(2600))
    width, k = 16384, 512
    kinds = ["normal", "bits", "ties", "negative", "neg_ties", "crowded"]
    L = np.full((rows, width), W.POISON, np.uint16)
    for i, kind in enumerate(kinds):
        L[i::len(kinds)] = _random_rows(rng, L[i::len(kinds)].shape[0], width, kind)
    pos = _sampled_positions_wg(width // 8)
    mis = np.arange(100, 1300, 97)                       # misjudged rows
    L[mis] = 0x3F00
    L[np.ix_(mis, pos)] = (0x4000 + np.arange(pos.size) % 0x700).astype(np.uint16)
    ovf = np.arange(150, rows, 211)                      # overflowing rows
    L[ovf] = W.f32_to_bf16_bits(np.abs(rng.standard_normal((ovf.size, width),
                                                           dtype=np.float32)) + 1)
    L[np.ix_(ovf, pos)] = 0x3C00
    lens = np.full(rows, width, np.int32)
    pick = rng.permutation(rows)
    free = np.setdiff1d(pick, np.concatenate([mis, ovf]), assume_unique=False)
    free = rng.permutation(free)
    ragged, short = free[:400], free[400:650]
    lens[ragged] = rng.integers(k + 1, width, size=ragged.size)
    lens[short] = rng.integers(0, k + 1, size=short.size)
    lens[free[650:660]] = [0, 1, k, k + 1, k + 7, width - 1, width - 8, -3, width + 9, 8 * 513 + 3]
    lens[-3:] = [k, width, k + 1]                        # the launch's last rows
    for r in range(rows):
        L[r, max(0, min(int(lens[r]), width)):] = W.POISON
    d = dict(logits=L, valid_len=lens, k=k, mode=0, width=width, pages=None, page_size=0)
    o = run_oracle(d)
    g, pc = run_gpu(d)
    assert_parity(d, g, o)
    paths = _paths(pc)
    print("paths", paths, flush=True)
    assert -9 not in paths
    assert np.all(pc[mis] == T.PATH_DIRECT_MISJUDGED), pc[mis]
    assert np.all(pc[ovf] == T.PATH_DIRECT_OVERFLOW), pc[ovf]
    assert paths.get(T.PATH_SHORT, 0) >= short.size
    assert paths.get(T.PATH_SAMPLED, 0) > rows // 2
    assert paths.get(T.PATH_SAMPLED_TIES, 0) > 0
    g, pc = run_gpu(d, force_direct=True)
    assert_parity(d, g, o)
    assert set(_paths(pc)) <= {T.PATH_DIRECT_FORCED, T.PATH_SHORT}


def test_many_block_rows():
    """Block rows, more than workgroups resident at once (the block
    throughput kernel): ragged lengths, -inf blocks, NaN blocks, short rows
    and a last group of fewer than 8 rows."""
    rng = np.random.Generator(np.random.PCG64(2603))
    rows, width, k = 2603, 16384, 512
    L = W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32))
    nblk = width // 8
    blk = L.reshape(rows, nblk, 8)
    blk[rng.random((rows, nblk)) < 0.02] = W.BF16_NEG_INF
    nan_rows = rng.choice(rows, 40, replace=False)
    blk[nan_rows, rng.integers(0, nblk, 40), rng.integers(0, 8, 40)] = 0xFFC1
    lens = (rng.integers(8 * k + 8, width + 1, size=rows) // 8 * 8).astype(np.int32)
    short = rng.choice(rows, 200, replace=False)
    lens[short] = rng.integers(0, 8 * k + 1, size=short.size)
    lens[-5:] = [width, 8 * k, 8 * k + 8, width - 5, 13]
    for r in range(rows):
        L[r, max(0, min(int(lens[r]), width)):] = W.POISON
    d = dict(logits=L, valid_len=lens, k=k, mode=W.MODE_BLOCK, width=width, pages=None,
             page_size=0)
    o = run_oracle(d)
    g, pc = run_gpu(d)
    assert_parity(d, g, o)
    paths = _paths(pc)
    print("paths", paths, flush=True)
    assert -9 not in paths
    assert paths.get(T.PATH_SAMPLED, 0) > rows // 2


@pytest.mark.parametrize("k", [64, 512])
@pytest.mark.parametrize("rows", [96, 600, 2600])
def test_short_rows_every_logit_sampled(k, rows):
    """Token rows of k + 1 .. 4096 logits (at most 512 vectors).  With every
    row resident (96 rows: a CU and 1024 threads a row; 600 rows: 512
    threads a row) every logit is a sample, and the cutoff is the key
    just below the exact k-th key unless the keys at or above it would fill
    more than half the survivor regions (then the tie pass): the sampled path
    or the tie pass, never the direct path, whatever the values, and mostly
    the sampled path.  The throughput kernel (2600 rows) keeps one sample a
    vector: the same results, on the sampled path, the tie pass or, for a
    tied row the samples misjudge, the direct path.  Constant rows of 0xFFFF
    (k-th key 0) take the direct path."""
    rng = np.random.Generator(np.random.PCG64(4000 + k + rows))
    width = 4096
    kinds = ["normal", "bits", "ties", "negative", "neg_ties", "crowded"]
    L = np.full((rows, width), W.POISON, np.uint16)
    for i, kind in enumerate(kinds):
        L[i::len(kinds)] = _random_rows(rng, L[i::len(kinds)].shape[0], width, kind)
    L[7] = 0x3F80                                          # a constant row
    L[8] = 0xFFFF                                          # every key 0
    lens = rng.integers(k + 1, width + 1, size=rows).astype(np.int32)
    lens[:6] = [k + 1, k + 7, 2048, 2049, 4095, 8 * 257 + 5]
    for r in range(rows):
        L[r, lens[r]:] = W.POISON
    d = dict(logits=L, valid_len=lens, k=k, mode=0, width=width, pages=None, page_size=0)
    o = run_oracle(d)
    g, pc = run_gpu(d)
    assert_parity(d, g, o)
    paths = _paths(pc)
    print("paths", paths, flush=True)
    assert pc[8] == T.PATH_DIRECT_MISJUDGED
    others = np.delete(pc, 8)
    if rows < 1000:   # every row resident: every logit sampled
        allowed = [T.PATH_SAMPLED, T.PATH_SAMPLED_TIES]
        assert (others == T.PATH_SAMPLED).mean() >= 0.6, _paths(others)
    else:             # one sample a vector: a tied short row may be misjudged
        allowed = [T.PATH_SAMPLED, T.PATH_SAMPLED_TIES, T.PATH_DIRECT_MISJUDGED]
    assert np.all(np.isin(others, allowed)), _paths(others)


@pytest.mark.parametrize("rows", [40, 2600])
def test_short_block_rows_every_block_sampled(rows):
    """Block rows of at most 512 blocks, where every block is sampled: the
    cutoff is the key just below the exact k-th block key, so no tie pass;
    ragged lengths, -inf and NaN blocks, and constant rows."""
    rng = np.random.Generator(np.random.PCG64(4100 + rows))
    width, k = 4096, 256
    L = W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32))
    blk = L.reshape(rows, width // 8, 8)
    blk[rng.random((rows, width // 8)) < 0.05] = W.BF16_NEG_INF
    blk[3, 17, 2] = 0x7FC1
    L[5] = 0x4000
    lens = rng.integers(8 * k + 1, width + 1, size=rows).astype(np.int32)
    lens[:3] = [8 * k + 1, width, width - 3]
    for r in range(rows):
        L[r, lens[r]:] = W.POISON
    d = dict(logits=L, valid_len=lens, k=k, mode=W.MODE_BLOCK, width=width, pages=None,
             page_size=0)
    o = run_oracle(d)
    g, pc = run_gpu(d)
    assert_parity(d, g, o)
    assert np.all(pc == T.PATH_SAMPLED), _paths(pc)


def _sampled_vectors_team(nvec, sv=1, nt=256):
    """Vectors every member of a token team samples for a row of nvec
    vectors (nvec > sv * nt): runs of 8 consecutive vectors, run r starting
    at line floor((2 r + 1) lines / (2 runs)) in 32.32 fixed point."""
    runs = sv * nt // 8
    step = ((nvec >> 3) << 32) // (2 * runs)
    si = np.arange(sv * nt)
    return ((((2 * (si >> 3) + 1) * step) >> 32) << 3) + (si & 7)


def test_team_skipped_ties_take_direct_path():
    """A wide row of one value X, but for 20 sampled logits above it: the
    samples above the cutoff (X) look plentiful, so the team does not collect
    keys equal to X, yet fewer than k keys lie above X.  The row must fall
    back to the direct path and stay exact."""
    width, k = 150000, 512
    L = np.full((2, width), 0x3F80, np.uint16)                    # 1.0
    pos = (_sampled_vectors_team(width // 8) * 8)[:20]
    L[:, pos] = (0x4000 + np.arange(20)).astype(np.uint16)         # 2.0 and up
    d = dict(logits=L, valid_len=np.full(2, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_DIRECT_MISJUDGED), pc


def test_team_ties_collected_when_needed():
    """A wide row of 0.5 with X = 1.0 at every 4th logit and 5 sampled logits
    above X: the samples give no assurance that k keys lie above the cutoff
    (X), and the keys at X (a quarter of the row) are too many to become
    survivors, so the team collects the keys equal to X and the row takes
    the tie pass (a row of 5 members: their capped tie lists fit the
    select's staging)."""
    width, k = 40000, 512
    L = np.full((2, width), 0x3F00, np.uint16)                    # 0.5
    L[:, ::4] = 0x3F80                                             # 1.0
    pos = (_sampled_vectors_team(width // 8) * 8 + 1)[:5]
    L[:, pos] = (0x4000 + np.arange(5)).astype(np.uint16)
    d = dict(logits=L, valid_len=np.full(2, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_SAMPLED_TIES), pc


def test_team_tied_cutoff_moves_below_the_ties():
    """A wide row of 0.5 with X = 1.0 at every 64th logit and 5 sampled
    logits above X: fewer than k keys lie above X, but the keys at X (1/64 of
    the row) fit the survivor regions, so the cutoff moves to the key below
    X, the keys at X are survivors and the row takes the plain sampled
    path, exact."""
    width, k = 150000, 512
    L = np.full((2, width), 0x3F00, np.uint16)                    # 0.5
    L[:, ::64] = 0x3F80                                            # 1.0
    pos = (_sampled_vectors_team(width // 8) * 8 + 1)[:5]
    L[:, pos] = (0x4000 + np.arange(5)).astype(np.uint16)
    d = dict(logits=L, valid_len=np.full(2, width, np.int32), k=k, mode=0, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_SAMPLED), pc


def test_team_member_region_overflow_takes_direct_path():
    """Block rows of 4500 blocks at k = 2048 go to the team path with more
    than half of every member's blocks above the cutoff: a member wave keeps
    more entries than its LDS region holds, reports the overflow, and the row
    takes the direct path, exact."""
    rng = np.random.Generator(np.random.PCG64(4500))
    width, k = 36000, 2048
    L = W.f32_to_bf16_bits(rng.standard_normal((2, width), dtype=np.float32))
    d = dict(logits=L, valid_len=np.full(2, width, np.int32), k=k, mode=1, width=width,
             pages=None, page_size=0)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert np.all(pc == T.PATH_DIRECT_OVERFLOW), pc


def test_team_scratch_reused_across_calls():
    """Consecutive team launches on one stream see clean scratch, also when
    a call has more rows than the one before it (regression: the control
    words once moved with the row count and overlapped old survivor lists)."""
    for rows in (2, 5):
        d = W.make(3, rows=rows, width=40000, seed=299 + rows)
        g, _ = run_gpu(d)
        assert_parity(d, g, run_oracle(d))
    d = W.make(3, rows=16, width=150000, seed=300)
    o = run_oracle(d)
    for _ in range(3):
        g, _ = run_gpu(d)
        assert_parity(d, g, o)
    d4 = W.make(4, rows=9, width=200000, seed=301)
    g, _ = run_gpu(d4)
    assert_parity(d4, g, run_oracle(d4))


def test_side_stream():
    d = W.make(2, rows=32, width=8192, seed=302)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g, _ = run_gpu(d, stream=s)
    assert_parity(d, g, run_oracle(d))
    d3 = W.make(3, rows=3, width=60000, seed=303)
    with torch.cuda.stream(s):
        g, _ = run_gpu(d3, stream=s)
    assert_parity(d3, g, run_oracle(d3))


def test_graph_replays():
    """Calls captured in one HIP graph (the row path with a block table, a
    token team and a block team) and replayed several times, with other
    eager calls and synchronizations between the replays: every replay's
    outputs match the oracle (the library records no memset, and its team
    scratch needs no clearing between calls)."""
    ds = [W.make(2, rows=48, width=16384, seed=401), W.make(3, rows=5, width=60000, seed=402),
          W.make(4, rows=6, width=150000, seed=403)]
    # eager work in between, on the same stream and scratch
    other = W.make(3, rows=7, width=50000, seed=404)
    os_ = [run_oracle(d) for d in ds]
    s = torch.cuda.Stream()
    dev = [_dev(d) for d in ds]

    def calls():
        return [T.topk_bf16_rows(L, VL, d["k"], d["mode"], block_table=P,
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
            for o in outs:
                o.fill_(-7)
            go, _ = run_gpu(other, stream=s)  # eager work on the same stream and scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        for d, o, ref in zip(ds, outs, os_):
            assert_parity(d, o.cpu().numpy(), ref)
    assert_parity(other, go, run_oracle(other))


def test_widest_rows():
    """Rows of 2^20 logits in token mode (the widest team) and block mode."""
    rng = np.random.Generator(np.random.PCG64(304))
    for mode, k in ((0, 2048), (1, 2048), (0, 1)):
        d = _make(rng, 2, 1 << 20, k, mode, "normal", lens=[1 << 20, 777777])
        g, pc = run_gpu(d)
        assert_parity(d, g, run_oracle(d))


def with_pages(d, P, rng, pad=3):
    """d with a per-row permuted block table of page size P (rows padded by
    `pad` unused entries past ceil(width / P))."""
    npg = -(-d["width"] // P)
    rows = d["logits"].shape[0]
    pages = np.full((rows, npg + pad), 1 << 30, np.int32)
    for r in range(rows):
        pages[r, :npg] = rng.permutation(npg)
    d = dict(d)
    d["pages"], d["page_size"] = pages, P
    return d


# (rows, width, k, mode, kind): launches with more rows than one team batch
# holds, so that later batches start at row0 > 0 (1024 rows a batch; 112
# rows of 2^20 tokens fill the scratch cap)
MULTI_BATCH = [(1100, 16392, 512, 0, "normal"), (120, 1 << 20, 2048, 0, "normal")]


@pytest.mark.parametrize("rows,width,k,mode,kind", MULTI_BATCH)
def test_team_multi_batch(rows, width, k, mode, kind):
    rng = np.random.Generator(np.random.PCG64(rows + width))
    lens = rng.integers(k + 1, width + 1, size=rows).astype(np.int32)
    lens[::7] = width
    lens[3::50] = k // 2                       # short rows in later batches too
    d = _make(rng, rows, width, k, mode, kind, lens=lens)
    print(f"multi-batch rows={rows} width={width}", flush=True)
    g, pc = run_gpu(d)
    assert_parity(d, g, run_oracle(d))
    assert -9 not in _paths(pc)


# page sizes other than 64 on one-workgroup rows (16384 tokens, 4096 blocks:
# the LDS copy of the table for P >= 16, the global table for P = 1) and on
# team rows, both modes
PAGE_CASES = [(P, width, mode) for P in (1, 16, 2048)
              for width, mode in ((16384, 0), (32768, 1), (100000, 0), (300000, 1))]


@pytest.mark.parametrize("P,width,mode", PAGE_CASES)
def test_page_sizes(P, width, mode):
    rng = np.random.Generator(np.random.PCG64(P * 31 + width + mode))
    k = 512 if mode == 0 else 1024
    lens = [width, width - 5, width // 2, k - 3, 3 * k]
    d = with_pages(_make(rng, 5, width, k, mode, "normal", lens=lens), P, rng)
    print(f"page size {P} width {width} mode {mode}", flush=True)
    for fd in (False, True):
        g, _ = run_gpu(d, force_direct=fd)
        assert_parity(d, g, run_oracle(d))
