"""The team scratch under HIP graph capture (topk_reserve_scratch): a
reserved scratch, or one a captured call used, is never replaced, so a
larger call fails with a reason instead of freeing memory a graph holds,
and the graph's replays stay correct; a call captured before any scratch
was set up fails without launching anything."""
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


def teardown_module(module):
    if T is not None and torch.cuda.is_available():
        torch.cuda.synchronize()
        T.release_scratch()


def _dev(d):
    L = torch.from_numpy(np.ascontiguousarray(d["logits"]).view(np.int16)).cuda()
    VL = torch.from_numpy(np.ascontiguousarray(d["valid_len"])).cuda()
    return L, VL


def _call(d, L, VL, out=None, stream=None):
    return T.topk_bf16_rows(L, VL, d["k"], d["mode"], width=d["width"], out=out, stream=stream)


def _assert_parity(d, got):
    want = oracle.topk(d["logits"], d["valid_len"], d["k"], d["mode"], width=d["width"],
                       threads=16)
    bad = check(oracle.default(), d, got, want)
    assert not bad, "\n".join(bad)


def _capture_and_check(small, s):
    L, VL = _dev(small)
    out = torch.empty((small["logits"].shape[0], small["k"]), dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _call(small, L, VL, out=out)
    return g, out, (L, VL)


def _replays_ok(g, out, small, s):
    for rep in range(2):
        with torch.cuda.stream(s):
            out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_parity(small, out.cpu().numpy())


def test_reserved_scratch_is_never_replaced():
    s = torch.cuda.Stream()
    small = W.make(4, rows=8, seed=611)      # 8 block rows of 2^20 logits: team rows
    big = W.make(4, rows=24, seed=612)
    T.reserve_scratch(8, small["width"], small["k"], small["mode"], stream=s)
    Lb, VLb = _dev(big)
    with pytest.raises(T.TopkError) as ei:   # a call never grows a reserved scratch
        with torch.cuda.stream(s):
            _call(big, Lb, VLb, stream=s)
    assert ei.value.status == -4 and "reserved" in str(ei.value), ei.value
    g, out, keep = _capture_and_check(small, s)
    _replays_ok(g, out, small, s)
    with pytest.raises(T.TopkError) as ei:   # nor, once captured, a reservation
        T.reserve_scratch(24, big["width"], big["k"], big["mode"], stream=s)
    assert ei.value.status == -4 and "captured graph" in str(ei.value), ei.value
    with pytest.raises(T.TopkError) as ei:
        with torch.cuda.stream(s):
            _call(big, Lb, VLb, stream=s)
    assert ei.value.status == -4, ei.value
    _replays_ok(g, out, small, s)            # the graph's scratch was not freed
    with torch.cuda.stream(s):               # a call within the reservation still runs
        got = _call(small, *keep, stream=s)
    torch.cuda.synchronize()
    _assert_parity(small, got.cpu().numpy())
    del g


def test_capture_pins_the_scratch():
    s = torch.cuda.Stream()
    small = W.make(4, rows=8, seed=621)
    big = W.make(4, rows=24, seed=622)
    L, VL = _dev(small)
    with torch.cuda.stream(s):
        _call(small, L, VL, stream=s)        # sets up the stream's scratch
    torch.cuda.synchronize()
    g, out, _ = _capture_and_check(small, s)
    Lb, VLb = _dev(big)
    with pytest.raises(T.TopkError) as ei:
        with torch.cuda.stream(s):
            _call(big, Lb, VLb, stream=s)
    assert ei.value.status == -4 and "captured graph" in str(ei.value), ei.value
    _replays_ok(g, out, small, s)
    del g


def test_capture_needs_scratch_set_up():
    s = torch.cuda.Stream()
    d = W.make(4, rows=4, seed=631)
    L, VL = _dev(d)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(T.TopkError) as ei:
        with torch.cuda.graph(g, stream=s):
            _call(d, L, VL)
    assert ei.value.status == -4 and "capture" in str(ei.value), ei.value
    del g
    torch.cuda.synchronize()
    with torch.cuda.stream(s):               # outside capture the same call runs
        got = _call(d, L, VL, stream=s)
    torch.cuda.synchronize()
    _assert_parity(d, got.cpu().numpy())
