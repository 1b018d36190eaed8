"""The entry point that allocates nothing (topk_bf16_rows_noalloc), through
the C ABI: its results meet the parity bar against the allocating entry
point's (topk_bf16_rows) and against the oracle, on consecutive calls that
reuse the library's fixed per-device scratch, the later ones smaller."""
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


def _run(fn, d):
    L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
    VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
    P = None if d.get("pages") is None else torch.from_numpy(d["pages"]).cuda()
    out = torch.full((L.shape[0], d["k"]), -7, dtype=torch.int32, device="cuda")
    fn(L, VL, d["k"], d["mode"], block_table=P, page_size=d.get("page_size") or 64,
       width=d["width"], out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _token_rows(rows, width, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    L = W.f32_to_bf16_bits(rng.standard_normal((rows, width), dtype=np.float32))
    lens = rng.integers(4096, width + 1, size=rows).astype(np.int32)
    lens[0] = width
    for r in range(rows):
        L[r, lens[r]:] = W.POISON
    return dict(logits=L, valid_len=lens, k=2048, mode=0, width=width, pages=None, page_size=0)


def test_noalloc_matches_allocating_entry_point():
    # 20 rows of 2^20 tokens: several batches of the fixed scratch; then
    # smaller calls on the same scratch: more one-workgroup rows than
    # resident workgroups, block rows, crowded rows with a block table,
    # one-workgroup rows, and many rows again
    cases = [("token 20 x 2^20", _token_rows(20, 1 << 20, 61)),
             ("many rows 3000 x 16384", W.make(5, rows=3000, seed=66)),
             ("block 12 x 2^20", W.make(4, rows=12, seed=62)),
             ("crowded 7 x 150000", W.make(3, rows=7, seed=63)),
             ("paged 40 x 16384", W.make(2, rows=40, seed=64)),
             ("many rows 2100 x 16384", W.make(5, rows=2100, seed=67))]
    for name, d in cases:
        print(f"no-alloc case {name}", flush=True)
        got = _run(T.topk_bf16_rows_noalloc, d)
        ref = _run(T.topk_bf16_rows, d)
        bad = check(oracle.default(), d, got, ref)
        assert not bad, f"{name} against topk_bf16_rows: " + "\n".join(bad)
        want = oracle.topk(d["logits"], d["valid_len"], d["k"], d["mode"], width=d["width"],
                           pages=d.get("pages"), page_size=d.get("page_size") or 64, threads=16)
        bad = check(oracle.default(), d, got, want)
        assert not bad, f"{name} against the oracle: " + "\n".join(bad)


def test_noalloc_requires_out():
    d = W.make(1, rows=2, width=1024, seed=65)
    L = torch.from_numpy(d["logits"].view(np.int16)).cuda()
    VL = torch.from_numpy(d["valid_len"]).cuda()
    with pytest.raises(ValueError):
        T.topk_bf16_rows_noalloc(L, VL, 8, 0)
