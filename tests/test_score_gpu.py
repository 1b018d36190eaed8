"""GPU parity of the FP8 and MXFP4 MQA indexer logits (topk_fp8_mqa_logits,
topk_mxfp4_mqa_logits) through
the C ABI, against the scorer oracle (oracle/score_oracle.c), and of the
selection they feed.

Two bars.  On inputs whose products sum exactly in FP32 ("narrow" bytes)
the matrix cores' dot products are exact, and every logit must equal the
oracle's definition bit for bit.  On full-range inputs ("wide" bytes) the
matrix cores' FP8 accumulation differs from the exact dot product (its order
and width are the hardware's; measured at most 2^-12.2 of the sum of the
products' magnitudes), so every logit must lie in the oracle's interval for
an allowance of 2^-10 of that sum.  The side array must be exactly the 8-key
maxima of the logits written, and the selection on them exactly the
oracle's top-k of those logits."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import score
import workloads as W
from checker import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

T = None
DELTA = 2.0 ** -10
SENTINEL = 0x7E57


def setup_module(module):
    global T
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_wise_amd as _T
    T = _T
    T.library()


def run_score(d, width=None):
    """The scorer on d's inputs; logits and tops start as SENTINEL."""
    width = d["width"] if width is None else width
    rows = d["q"].shape[0]
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(d["q"]).to(dev)
    w = torch.from_numpy(d["w"].view(np.int16)).to(dev)
    keys = torch.from_numpy(d["keys"]).to(dev)
    ks = torch.from_numpy(d["key_scale"]).to(dev)
    vl = torch.from_numpy(d["valid_len"]).to(dev)
    nv = (width + 7) // 8
    logits = torch.full((rows, max(8, -(-width // 8) * 8)), SENTINEL, dtype=torch.int16, device=dev)
    tops = torch.full((rows, max(8, -(-nv // 8) * 8)), SENTINEL, dtype=torch.int16, device=dev)
    T.fp8_mqa_logits(q, w, keys, ks, vl, d["qpr"], width=width, logits=logits, tops=tops)
    torch.cuda.synchronize()
    return logits.cpu().numpy().view(np.uint16), tops.cpu().numpy().view(np.uint16)


def oracle_row(d, t, delta, cols=None):
    """(exact, lo, hi) of row t over its valid keys (or the given columns)."""
    so = score.load()
    r = t // d["qpr"]
    v = max(0, min(int(d["valid_len"][t]), d["width"]))
    idx = np.arange(v) if cols is None else np.asarray(cols)
    return so.mqa_logits(d["q"][t:t + 1], d["w"][t:t + 1], d["keys"][r][idx],
                         d["key_scale"][r][idx], delta)


def _vkey(b):
    b = np.asarray(b, np.uint16).astype(np.uint32)
    return np.where(b & 0x8000, b ^ 0xFFFF, b ^ 0x8000)


def check_untouched_and_tops(d, logits, tops):
    width = d["width"]
    for t in range(logits.shape[0]):
        v = max(0, min(int(d["valid_len"][t]), width))
        nv = (v + 7) // 8
        assert np.all(logits[t, v:] == SENTINEL), f"row {t}: written past its length"
        assert np.all(tops[t, nv:] == SENTINEL), f"row {t}: maxima written past the length"
        want = oracle.vector_maxima(logits[t:t + 1, :max(v, 1)], np.array([v], np.int32),
                                    max(v, 1))[0][:nv]
        assert np.array_equal(tops[t, :nv], want), f"row {t}: maxima of the logits differ"


@pytest.mark.parametrize("requests,qpr,width,ks", [(2, 3, 700, 720), (3, 1, 257, 257),
                                                    (1, 2, 1031, 1100)])
def test_narrow_inputs_bit_exact(requests, qpr, width, ks):
    d = W.make_score(requests, qpr, width, "narrow", seed=width, key_stride=ks)
    print(f"score narrow requests={requests} qpr={qpr} width={width}", flush=True)
    logits, tops = run_score(d)
    for t in range(d["q"].shape[0]):
        v = max(0, min(int(d["valid_len"][t]), width))
        ex, lo, hi = oracle_row(d, t, 0.0)
        assert np.array_equal(lo, ex) and np.array_equal(hi, ex)
        bad = np.nonzero(logits[t, :v] != ex[0])[0]
        assert bad.size == 0, f"row {t}: {bad.size} logits differ, first at key {bad[:3]}"
    check_untouched_and_tops(d, logits, tops)


@pytest.mark.parametrize("requests,qpr,width", [(3, 2, 1000), (2, 1, 4096)])
def test_wide_inputs_within_the_interval(requests, qpr, width):
    d = W.make_score(requests, qpr, width, "wide", seed=width + 7)
    print(f"score wide requests={requests} qpr={qpr} width={width}", flush=True)
    logits, tops = run_score(d)
    same = total = 0
    for t in range(d["q"].shape[0]):
        v = max(0, min(int(d["valid_len"][t]), width))
        ex, lo, hi = oracle_row(d, t, DELTA)
        g = _vkey(logits[t, :v])
        out = np.nonzero((g < _vkey(lo[0])) | (g > _vkey(hi[0])))[0]
        assert out.size == 0, f"row {t}: {out.size} logits outside the interval, first {out[:3]}"
        same += int((logits[t, :v] == ex[0]).sum())
        total += v
    print(f"  {same} of {total} logits equal the exact dot products' ({same / max(total, 1):.3f})")
    check_untouched_and_tops(d, logits, tops)


def test_lengths_and_many_verify_rows():
    """Valid lengths 0, 1, 7, 8, 9, 255, 256, 257, the width, past it and
    negative (clamped); and 8 verify rows to a request."""
    d = W.make_score(10, 1, 600, "narrow", seed=3, key_stride=640)
    d["valid_len"] = np.array([0, 1, 7, 8, 9, 255, 256, 257, 600, 611], np.int32)
    logits, tops = run_score(d)
    for t in range(10):
        v = max(0, min(int(d["valid_len"][t]), 600))
        ex, _, _ = oracle_row(d, t, 0.0)
        assert np.array_equal(logits[t, :v], ex[0]), f"row {t} (v={v})"
    check_untouched_and_tops(d, logits, tops)
    d = W.make_score(2, 8, 333, "narrow", seed=4)
    d["valid_len"][3] = -3
    logits, tops = run_score(d)
    for t in range(16):
        v = max(0, min(int(d["valid_len"][t]), 333))
        ex, _, _ = oracle_row(d, t, 0.0)
        assert np.array_equal(logits[t, :v], ex[0]), f"qpr 8 row {t} (v={v})"
    check_untouched_and_tops(d, logits, tops)


@pytest.mark.parametrize("kind", ["narrow", "wide"])
def test_scores_feed_the_selection(kind):
    """The scorer's logits and maxima into topk_bf16_rows_tops: the exact
    top-k of the logits written (k = 512 over rows of 4096 .. 20000 keys)."""
    d = W.make_score(6, 2, 20000, kind, seed=11)
    logits, tops = run_score(d)
    rows = logits.shape[0]
    dev = torch.device("cuda", 0)
    L = torch.from_numpy(logits.view(np.int16)).to(dev)
    VL = torch.from_numpy(d["valid_len"]).to(dev)
    tp = torch.from_numpy(tops.view(np.int16)).to(dev)
    pc = torch.full((rows,), -9, dtype=torch.int32, device=dev)
    k = 512
    out = T.topk_bf16_rows_tops(L, VL, k, tp, 0, width=d["width"], path_codes=pc)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    sel = dict(logits=logits, valid_len=d["valid_len"], k=k, mode=0, width=d["width"],
               pages=None, page_size=0)
    o = oracle.topk(logits, d["valid_len"], k, 0, width=d["width"], threads=16)
    bad = check(oracle.default(), sel, g, o)
    assert not bad, "\n".join(bad)
    assert np.all(pc.cpu().numpy() == T.PATH_TOPS), pc.cpu().numpy()


def test_full_size_sampled():
    """The benchmark's scorer workload (64 requests x 150000 keys, one
    verify row each): 4000 sampled logits in the oracle's interval, and every
    row's maxima those of its logits."""
    c = W.SCORE_CONFIG
    d = W.make_score(c["requests"], c["qpr"], c["width"], "wide", seed=0, ragged=True)
    print(f"score full size {c['name']}", flush=True)
    logits, tops = run_score(d)
    rng = np.random.Generator(np.random.PCG64(5))
    rows = d["q"].shape[0]
    for t in range(rows):
        v = max(0, min(int(d["valid_len"][t]), d["width"]))
        cols = np.sort(rng.choice(v, size=min(v, 4000 // rows), replace=False))
        ex, lo, hi = oracle_row(d, t, DELTA, cols)
        g = _vkey(logits[t, cols])
        assert np.all((g >= _vkey(lo[0])) & (g <= _vkey(hi[0]))), f"row {t}"
    check_untouched_and_tops(d, logits, tops)


# -- MXFP4 (topk_mxfp4_mqa_logits).  The matrix cores' block-scaled sums are
# exact when each dot product's products share one power of two ("uniform"
# scales: a head's four blocks alike and a key's four alike), and then
# every logit must equal the oracle's; with a scale per block they may lose
# the last FP32 bits (measured at most 2^-23.5 of the sum of the products'
# magnitudes), and every logit must lie in the oracle's interval for an
# allowance of 2^-20 of that sum.
DELTA4 = 2.0 ** -20


def run_score_fp4(d, width=None):
    width = d["width"] if width is None else width
    rows = d["q"].shape[0]
    dev = torch.device("cuda", 0)
    args = [torch.from_numpy(d[k]).to(dev) for k in ("q", "q_scale")]
    w = torch.from_numpy(d["w"].view(np.int16)).to(dev)
    keys = torch.from_numpy(d["keys"]).to(dev)
    ks = torch.from_numpy(d["key_scale"]).to(dev)
    vl = torch.from_numpy(d["valid_len"]).to(dev)
    nv = (width + 7) // 8
    logits = torch.full((rows, max(8, -(-width // 8) * 8)), SENTINEL, dtype=torch.int16, device=dev)
    tops = torch.full((rows, max(8, -(-nv // 8) * 8)), SENTINEL, dtype=torch.int16, device=dev)
    T.mxfp4_mqa_logits(args[0], args[1], w, keys, ks, vl, d["qpr"], width=width, logits=logits,
                       tops=tops)
    torch.cuda.synchronize()
    return logits.cpu().numpy().view(np.uint16), tops.cpu().numpy().view(np.uint16)


def oracle_row_fp4(d, t, delta, cols=None):
    so = score.load()
    r = t // d["qpr"]
    v = max(0, min(int(d["valid_len"][t]), d["width"]))
    idx = np.arange(v) if cols is None else np.asarray(cols)
    return so.mxfp4_logits(d["q"][t:t + 1], d["q_scale"][t:t + 1], d["w"][t:t + 1],
                           d["keys"][r][idx], d["key_scale"][r][idx], delta)


@pytest.mark.parametrize("requests,qpr,width,ks", [(2, 3, 700, 720), (3, 1, 257, 257),
                                                    (1, 2, 1031, 1100)])
def test_mxfp4_uniform_scales_bit_exact(requests, qpr, width, ks):
    d = W.make_score_mxfp4(requests, qpr, width, "uniform", seed=width, key_stride=ks)
    print(f"score mxfp4 uniform requests={requests} qpr={qpr} width={width}", flush=True)
    logits, tops = run_score_fp4(d)
    for t in range(d["q"].shape[0]):
        v = max(0, min(int(d["valid_len"][t]), width))
        ex, lo, hi = oracle_row_fp4(d, t, 0.0)
        assert np.array_equal(lo, ex) and np.array_equal(hi, ex)
        bad = np.nonzero(logits[t, :v] != ex[0])[0]
        assert bad.size == 0, f"row {t}: {bad.size} logits differ, first at key {bad[:3]}"
    check_untouched_and_tops(d, logits, tops)


@pytest.mark.parametrize("requests,qpr,width", [(3, 2, 1000), (2, 1, 4096)])
def test_mxfp4_block_scales_within_the_interval(requests, qpr, width):
    d = W.make_score_mxfp4(requests, qpr, width, "blocks", seed=width + 7)
    print(f"score mxfp4 blocks requests={requests} qpr={qpr} width={width}", flush=True)
    logits, tops = run_score_fp4(d)
    same = total = 0
    for t in range(d["q"].shape[0]):
        v = max(0, min(int(d["valid_len"][t]), width))
        ex, lo, hi = oracle_row_fp4(d, t, DELTA4)
        g = _vkey(logits[t, :v])
        out = np.nonzero((g < _vkey(lo[0])) | (g > _vkey(hi[0])))[0]
        assert out.size == 0, f"row {t}: {out.size} logits outside the interval, first {out[:3]}"
        same += int((logits[t, :v] == ex[0]).sum())
        total += v
    print(f"  {same} of {total} logits equal the exact dot products' ({same / max(total, 1):.4f})")
    check_untouched_and_tops(d, logits, tops)


def test_mxfp4_lengths_and_many_verify_rows():
    d = W.make_score_mxfp4(10, 1, 600, "uniform", seed=3, key_stride=640)
    d["valid_len"] = np.array([0, 1, 7, 8, 9, 255, 256, 257, 600, 611], np.int32)
    logits, tops = run_score_fp4(d)
    for t in range(10):
        v = max(0, min(int(d["valid_len"][t]), 600))
        ex, _, _ = oracle_row_fp4(d, t, 0.0)
        assert np.array_equal(logits[t, :v], ex[0]), f"row {t} (v={v})"
    check_untouched_and_tops(d, logits, tops)
    d = W.make_score_mxfp4(2, 8, 333, "uniform", seed=4)
    d["valid_len"][3] = -3
    logits, tops = run_score_fp4(d)
    for t in range(16):
        v = max(0, min(int(d["valid_len"][t]), 333))
        ex, _, _ = oracle_row_fp4(d, t, 0.0)
        assert np.array_equal(logits[t, :v], ex[0]), f"qpr 8 row {t} (v={v})"
    check_untouched_and_tops(d, logits, tops)


def test_mxfp4_scores_feed_the_selection():
    d = W.make_score_mxfp4(6, 2, 20000, "blocks", seed=12)
    logits, tops = run_score_fp4(d)
    rows = logits.shape[0]
    dev = torch.device("cuda", 0)
    L = torch.from_numpy(logits.view(np.int16)).to(dev)
    VL = torch.from_numpy(d["valid_len"]).to(dev)
    tp = torch.from_numpy(tops.view(np.int16)).to(dev)
    pc = torch.full((rows,), -9, dtype=torch.int32, device=dev)
    k = 512
    out = T.topk_bf16_rows_tops(L, VL, k, tp, 0, width=d["width"], path_codes=pc)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    sel = dict(logits=logits, valid_len=d["valid_len"], k=k, mode=0, width=d["width"],
               pages=None, page_size=0)
    o = oracle.topk(logits, d["valid_len"], k, 0, width=d["width"], threads=16)
    bad = check(oracle.default(), sel, g, o)
    assert not bad, "\n".join(bad)
    assert np.all(pc.cpu().numpy() == T.PATH_TOPS), pc.cpu().numpy()


def test_mxfp4_full_size_sampled():
    """The benchmark's MXFP4 workload (64 requests x 150000 keys): 4000
    sampled logits in the oracle's interval, every row's maxima those of
    its logits."""
    c = W.SCORE_FP4_CONFIG
    d = W.make_score_mxfp4(c["requests"], c["qpr"], c["width"], "blocks", seed=0)
    print(f"score full size {c['name']}", flush=True)
    logits, tops = run_score_fp4(d)
    rng = np.random.Generator(np.random.PCG64(6))
    rows = d["q"].shape[0]
    for t in range(rows):
        v = max(0, min(int(d["valid_len"][t]), d["width"]))
        cols = np.sort(rng.choice(v, size=min(v, 4000 // rows), replace=False))
        ex, lo, hi = oracle_row_fp4(d, t, DELTA4, cols)
        g = _vkey(logits[t, cols])
        assert np.all((g >= _vkey(lo[0])) & (g <= _vkey(hi[0]))), f"row {t}"
    check_untouched_and_tops(d, logits, tops)


def test_scorers_in_a_replayed_graph():
    """Both scorers and the selection after them, captured into one HIP
    graph and replayed three times with eager work and synchronizations in
    between: every replay's logits, maxima and selection equal the eager
    calls' (the scorers allocate nothing and record no memset)."""
    dev = torch.device("cuda", 0)
    d8 = W.make_score(2, 2, 3000, "wide", seed=31)
    d4 = W.make_score_mxfp4(2, 2, 3000, "blocks", seed=32)
    stream = torch.cuda.Stream(dev)
    outs = {}
    bufs = {}
    for name, d in (("fp8", d8), ("fp4", d4)):
        rows, width = d["q"].shape[0], d["width"]
        b = dict(q=torch.from_numpy(d["q"]).to(dev), w=torch.from_numpy(d["w"].view(np.int16)).to(dev),
                 keys=torch.from_numpy(d["keys"]).to(dev), ks=torch.from_numpy(d["key_scale"]).to(dev),
                 vl=torch.from_numpy(d["valid_len"]).to(dev),
                 logits=torch.zeros((rows, -(-width // 8) * 8), dtype=torch.int16, device=dev),
                 tops=torch.zeros((rows, 384), dtype=torch.int16, device=dev),
                 out=torch.zeros((rows, 256), dtype=torch.int32, device=dev))
        if name == "fp4":
            b["qs"] = torch.from_numpy(d["q_scale"]).to(dev)
        bufs[name] = (d, b)

    def calls():
        for name, (d, b) in bufs.items():
            if name == "fp4":
                T.mxfp4_mqa_logits(b["q"], b["qs"], b["w"], b["keys"], b["ks"], b["vl"], d["qpr"],
                                   width=d["width"], logits=b["logits"], tops=b["tops"],
                                   stream=stream)
            else:
                T.fp8_mqa_logits(b["q"], b["w"], b["keys"], b["ks"], b["vl"], d["qpr"],
                                 width=d["width"], logits=b["logits"], tops=b["tops"],
                                 stream=stream)
            T.topk_bf16_rows_tops(b["logits"], b["vl"], 256, b["tops"], 0, width=d["width"],
                                  out=b["out"], stream=stream)

    def snapshot():
        # the selection's unique part: each row's selected keys as a sorted
        # multiset (ties at the k-th key may be taken in any order), after
        # checking that its indices are distinct and valid
        torch.cuda.synchronize()
        res = {}
        for n, (d, b) in bufs.items():
            lg = b["logits"].cpu().numpy().view(np.uint16)
            out = b["out"].cpu().numpy()
            keys = []
            for t in range(out.shape[0]):
                v = int(d["valid_len"][t])
                idx = out[t]
                assert np.all((idx >= 0) & (idx < v)) and np.unique(idx).size == idx.size, (n, t)
                keys.append(np.sort(_vkey(lg[t, idx])))
            res[n] = (b["logits"].cpu().clone(), b["tops"].cpu().clone(), np.array(keys))
        return res

    def poison():
        for n, (d, b) in bufs.items():
            b["logits"].fill_(0x7E57)
            b["tops"].fill_(0x7E57)
            b["out"].fill_(-7)
        torch.cuda.synchronize()

    poison()
    with torch.cuda.stream(stream):
        calls()
    want = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    for rep in range(3):
        poison()
        with torch.cuda.stream(stream):
            graph.replay()
        got = snapshot()
        for n in want:
            assert torch.equal(got[n][0], want[n][0]), f"replay {rep}: {n} logits differ"
            assert torch.equal(got[n][1], want[n][1]), f"replay {rep}: {n} maxima differ"
            assert np.array_equal(got[n][2], want[n][2]), f"replay {rep}: {n} selection differs"
        with torch.cuda.stream(stream):
            calls()  # eager work between the replays
        torch.cuda.synchronize()
    del graph


@pytest.mark.parametrize("fp4", [False, True])
def test_odd_strides_and_offsets(fp4):
    """Logits and maxima rows of odd strides at an odd element offset (the
    stores are 2-byte), keys in a slot wider than the width: the logits
    equal the oracle's, nothing past a row's length or between rows is
    written."""
    width, ks = 777, 900
    d = (W.make_score_mxfp4(3, 1, width, "uniform", seed=41, key_stride=ks) if fp4
         else W.make_score(3, 1, width, "narrow", seed=41, key_stride=ks))
    rows = d["q"].shape[0]
    dev = torch.device("cuda", 0)
    lstride, tstride = width + 5, (width + 7) // 8 + 3
    lbuf = torch.full((rows * lstride + 2,), SENTINEL, dtype=torch.int16, device=dev)
    tbuf = torch.full((rows * tstride + 2,), SENTINEL, dtype=torch.int16, device=dev)
    logits = lbuf[1:1 + rows * lstride].view(rows, lstride)
    tops = tbuf[1:1 + rows * tstride].view(rows, tstride)
    args = [torch.from_numpy(d["q"]).to(dev)]
    if fp4:
        args.append(torch.from_numpy(d["q_scale"]).to(dev))
    args += [torch.from_numpy(d["w"].view(np.int16)).to(dev), torch.from_numpy(d["keys"]).to(dev),
             torch.from_numpy(d["key_scale"]).to(dev), torch.from_numpy(d["valid_len"]).to(dev)]
    fn = T.mxfp4_mqa_logits if fp4 else T.fp8_mqa_logits
    fn(*args, d["qpr"], width=width, logits=logits, tops=tops)
    torch.cuda.synchronize()
    lb = lbuf.cpu().numpy().view(np.uint16)
    tb = tbuf.cpu().numpy().view(np.uint16)
    assert lb[0] == SENTINEL and lb[-1] == SENTINEL and tb[0] == SENTINEL and tb[-1] == SENTINEL
    lg = lb[1:1 + rows * lstride].reshape(rows, lstride)
    tp = tb[1:1 + rows * tstride].reshape(rows, tstride)
    for t in range(rows):
        v = max(0, min(int(d["valid_len"][t]), width))
        ex, _, _ = oracle_row_fp4(d, t, 0.0) if fp4 else oracle_row(d, t, 0.0)
        assert np.array_equal(lg[t, :v], ex[0]), f"row {t}"
        assert np.all(lg[t, v:] == SENTINEL), f"row {t}: written past its length"
        nv = (v + 7) // 8
        want = oracle.vector_maxima(ex, np.array([v], np.int32), max(v, 1))[0][:nv]
        assert np.array_equal(tp[t, :nv], want) and np.all(tp[t, nv:] == SENTINEL), f"row {t} maxima"
