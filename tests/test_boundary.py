"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import exact_row_wise_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libtopk.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(topk_[a-z0-9_]+)\s*\(", text)))


# every header under include/ and the library that exports what it declares
LIBRARIES = {"libtopk.h": "libtopk.so", "libtopk_probe.h": "libtopk_probe.so"}


def test_every_header_has_a_library():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == sorted(LIBRARIES)


@pytest.mark.parametrize("header,lib", sorted(LIBRARIES.items()))
def test_libraries_export_their_headers(header, lib):
    so = ctypes.CDLL(os.path.join(os.path.dirname(T.library_path()), lib))
    names = declared_functions(os.path.join(ROOT, "include", header))
    assert names
    for name in names:
        assert hasattr(so, name), f"{lib} does not export {name}"


@pytest.mark.parametrize("args,status", [
    ((16, -16), -1), ((16, 24), -1), ((24, 32), -1), ((None, 32), -1), ((16, 0), 0),
    ((16, (1 << 40) + 16), -1),
])
def test_probe_rejects_bad_arguments(args, status):
    """Argument errors are found before any launch (no GPU needed)."""
    lib = T.probe_library()
    src, nbytes = args
    assert lib.topk_probe_stream_read(src, nbytes, 64, None) == status


def test_header_declares_entry_points():
    names = declared_functions()
    assert "topk_bf16_rows" in names and "topk_status_string" in names
    assert "topk_bf16_rows_ordered" in names and "topk_bf16_rows_ordered_ex" in names
    assert "topk_bf16_rows_noalloc" in names
    assert "topk_bf16_rows_tops" in names and "topk_bf16_vector_maxima" in names
    assert "topk_fp8_mqa_logits" in names and "topk_mxfp4_mqa_logits" in names
    assert len(names) >= 12


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(T.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"libtopk.so does not export {name}"


def test_status_strings():
    assert T.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert T.status_string(s) and T.status_string(s) != "unknown status"
    assert T.status_string(12345) == "unknown status"


def _call(**kw):
    lib = T.library()
    a = dict(logits=16, row_stride=16, valid_len=64, rows=4, width=16, k=8, mode=0,
             bt=None, out=128, stream=None)
    a.update(kw)
    return lib.topk_bf16_rows(a["logits"], a["row_stride"], a["valid_len"], a["rows"],
                              a["width"], a["k"], a["mode"], a["bt"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), -1), (dict(k=2049), -1), (dict(mode=2), -1), (dict(rows=-1), -1),
    (dict(width=-1), -1), (dict(width=(1 << 20) + 8, row_stride=(1 << 20) + 8), -1),
    (dict(row_stride=8), -1), (dict(row_stride=20), -2), (dict(logits=None), -1),
    (dict(valid_len=None), -1), (dict(out=None), -1), (dict(logits=24), -2),
    (dict(out=130), -2),
])
def test_rejects_bad_arguments(kw, status):
    assert _call(**kw) == status
    assert T.library().topk_last_error()


def test_rows_zero_is_a_noop():
    assert _call(rows=0, logits=None, valid_len=None, out=None) == 0


def test_bad_block_table():
    bt = T._binding._BlockTable(None, 1, 64)
    assert _call(bt=ctypes.pointer(bt)) == -1
    bt = T._binding._BlockTable(256, 1, 48)          # not a power of two
    assert _call(bt=ctypes.pointer(bt)) == -1
    bt = T._binding._BlockTable(256, 0, 8)           # rows too short for width 16
    assert _call(bt=ctypes.pointer(bt)) == -1


def _call_ordered(**kw):
    lib = T.library()
    a = dict(logits=16, row_stride=16, valid_len=64, rows=4, width=16, k=8, mode=0,
             bt=None, out=128, valid=256, ids=512, stream=None)
    a.update(kw)
    return lib.topk_bf16_rows_ordered(a["logits"], a["row_stride"], a["valid_len"], a["rows"],
                                      a["width"], a["k"], a["mode"], a["bt"], a["out"],
                                      a["valid"], a["ids"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), -1), (dict(k=2049), -1), (dict(mode=2), -1), (dict(row_stride=20), -2),
    (dict(out=None), -1), (dict(valid=258), -2), (dict(ids=514), -2), (dict(logits=24), -2),
])
def test_ordered_rejects_bad_arguments(kw, status):
    """The ordered entry point checks its arguments as the plain one does,
    and also the alignment of valid and ids (both may be NULL)."""
    assert _call_ordered(**kw) == status
    assert T.library().topk_last_error()


def test_ordered_rows_zero_is_a_noop():
    assert _call_ordered(rows=0, logits=None, valid_len=None, out=None, valid=None,
                         ids=None) == 0


def _call_tops(**kw):
    lib = T.library()
    a = dict(logits=16, row_stride=16, valid_len=64, rows=4, width=16, k=8, mode=0,
             tops=1024, tops_stride=8, bt=None, out=128, opts=None, stream=None)
    a.update(kw)
    return lib.topk_bf16_rows_tops(a["logits"], a["row_stride"], a["valid_len"], a["rows"],
                                   a["width"], a["k"], a["mode"], a["tops"], a["tops_stride"],
                                   a["bt"], a["out"], a["opts"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), -1), (dict(mode=2), -1), (dict(row_stride=20), -2), (dict(out=None), -1),
    (dict(tops=None), -1), (dict(tops=1032), -2), (dict(tops_stride=4), -2),
    (dict(tops_stride=0), -1), (dict(width=200, row_stride=200, tops_stride=24), -1),
])
def test_tops_rejects_bad_arguments(kw, status):
    """The entry point given vector maxima checks them (16-byte aligned rows
    of at least ceil(width / 8) entries) besides the usual arguments."""
    assert _call_tops(**kw) == status
    assert T.library().topk_last_error()


def test_tops_not_needed_in_block_mode_or_for_no_rows():
    assert _call_tops(rows=0, logits=None, valid_len=None, out=None, tops=None) == 0
    # block mode ignores the maxima: the same checks as topk_bf16_rows, and
    # a null side array is accepted (nothing is launched for these bad k)
    assert _call_tops(mode=1, tops=None, k=0) == -1


def _call_maxima(**kw):
    lib = T.library()
    a = dict(logits=16, row_stride=16, valid_len=64, rows=4, width=16, tops=1024,
             tops_stride=8, stream=None)
    a.update(kw)
    return lib.topk_bf16_vector_maxima(a["logits"], a["row_stride"], a["valid_len"], a["rows"],
                                       a["width"], a["tops"], a["tops_stride"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), -1), (dict(width=-1), -1), (dict(row_stride=8), -1),
    (dict(row_stride=20), -2), (dict(logits=None), -1), (dict(valid_len=None), -1),
    (dict(logits=24), -2), (dict(tops=None), -1), (dict(tops=1026), -2),
    (dict(tops_stride=12), -2), (dict(width=200, row_stride=200, tops_stride=16), -1),
])
def test_vector_maxima_rejects_bad_arguments(kw, status):
    assert _call_maxima(**kw) == status
    assert T.library().topk_last_error()


def test_vector_maxima_nothing_to_do():
    assert _call_maxima(rows=0, logits=None, valid_len=None, tops=None) == 0
    assert _call_maxima(width=0, logits=None, valid_len=None, tops=None) == 0


@pytest.mark.parametrize("args,status", [
    ((4, 1 << 20, 0, 0, 0), -1), ((4, 1 << 20, 8, 2, 0), -1), ((-1, 1 << 20, 8, 0, 0), -1),
    ((4, (1 << 20) + 8, 8, 0, 0), -1), ((4, -1, 8, 0, 0), -1),
])
def test_reserve_rejects_bad_arguments(args, status):
    assert T.library().topk_reserve_scratch(*args, None) == status
    assert T.library().topk_last_error()


def test_reserve_nothing_for_one_workgroup_rows():
    # rows that fit one workgroup take no scratch: nothing is reserved (and
    # no HIP call is made, so this runs without a GPU)
    lib = T.library()
    assert lib.topk_reserve_scratch(1000, 16384, 2048, 0, 0, None) == 0
    assert lib.topk_reserve_scratch(1000, 32768, 2048, 1, 1, None) == 0
    assert lib.topk_reserve_scratch(0, 1 << 20, 2048, 0, 0, None) == 0


def _call_score(**kw):
    lib = T.library()
    a = dict(q=4096, w=64, keys=8192, key_scale=7, key_stride=100, valid_len=64, rows=4, qpr=2,
             width=100, logits=1024, logits_stride=100, tops=2048, tops_stride=16, stream=None)
    a.update(kw)
    return lib.topk_fp8_mqa_logits(a["q"], a["w"], a["keys"], a["key_scale"], a["key_stride"],
                                   a["valid_len"], a["rows"], a["qpr"], a["width"], a["logits"],
                                   a["logits_stride"], a["tops"], a["tops_stride"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-2), -1), (dict(qpr=0), -1), (dict(qpr=9), -1), (dict(rows=5), -1),
    (dict(width=-1), -1), (dict(width=(1 << 20) + 1), -1), (dict(q=None), -1),
    (dict(w=None), -1), (dict(keys=None), -1), (dict(key_scale=None), -1),
    (dict(valid_len=None), -1), (dict(logits=None), -1), (dict(tops=None), -1),
    (dict(key_stride=99), -1), (dict(logits_stride=99), -1), (dict(tops_stride=12), -1),
    (dict(q=4104), -2), (dict(keys=8200), -2), (dict(w=66), -2), (dict(logits=1025), -2),
    (dict(tops=2049), -2),
])
def test_score_rejects_bad_arguments(kw, status):
    assert _call_score(**kw) == status
    assert T.library().topk_last_error()


def test_score_nothing_to_do():
    assert _call_score(rows=0, q=None, w=None, keys=None, key_scale=None, valid_len=None,
                       logits=None, tops=None) == 0
    assert _call_score(width=0, q=None, w=None, keys=None, key_scale=None, valid_len=None,
                       logits=None, tops=None) == 0


def _call_score_fp4(**kw):
    lib = T.library()
    a = dict(q=4096, q_scale=5, w=64, keys=8192, key_scale=7, key_stride=100, valid_len=64,
             rows=4, qpr=2, width=100, logits=1024, logits_stride=100, tops=2048, tops_stride=16,
             stream=None)
    a.update(kw)
    return lib.topk_mxfp4_mqa_logits(a["q"], a["q_scale"], a["w"], a["keys"], a["key_scale"],
                                     a["key_stride"], a["valid_len"], a["rows"], a["qpr"],
                                     a["width"], a["logits"], a["logits_stride"], a["tops"],
                                     a["tops_stride"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-2), -1), (dict(qpr=0), -1), (dict(qpr=9), -1), (dict(rows=5), -1),
    (dict(width=-1), -1), (dict(width=(1 << 20) + 1), -1), (dict(q=None), -1),
    (dict(q_scale=None), -1), (dict(w=None), -1), (dict(keys=None), -1),
    (dict(key_scale=None), -1), (dict(valid_len=None), -1), (dict(logits=None), -1),
    (dict(tops=None), -1), (dict(key_stride=99), -1), (dict(logits_stride=99), -1),
    (dict(tops_stride=12), -1), (dict(q=4104), -2), (dict(keys=8200), -2), (dict(w=66), -2),
    (dict(logits=1025), -2), (dict(tops=2049), -2),
])
def test_score_mxfp4_rejects_bad_arguments(kw, status):
    assert _call_score_fp4(**kw) == status
    assert T.library().topk_last_error()


def test_score_mxfp4_nothing_to_do():
    assert _call_score_fp4(rows=0, q=None, q_scale=None, w=None, keys=None, key_scale=None,
                           valid_len=None, logits=None, tops=None) == 0
    assert _call_score_fp4(width=0, q=None, q_scale=None, w=None, keys=None, key_scale=None,
                           valid_len=None, logits=None, tops=None) == 0
