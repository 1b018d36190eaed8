"""ctypes wrapper of ``topk_oracle.c`` (test infrastructure only).

Each method names the C function it calls; the C source cites the passages
of the pages it follows.  Nothing here computes keys or selections itself.

``Oracle(path)`` wraps one compiled copy of the C source, so that tests can
also load a copy built from a deliberately altered source (a planted
mistake) and check that the pins reject it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MODE_TOKEN = 0
MODE_BLOCK = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "topk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_default = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)


def lib_path() -> str:
    return _LIB


def compile_source(src: str, dst: str, libs=()) -> str:
    """gcc -O2 -shared: one C file into one shared library."""
    tmp = dst + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, *libs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)
    return dst


def build() -> str:
    """Compile oracle/topk_oracle.c into oracle/liboracle.so, and the
    scorer oracle (oracle/score_oracle.c) beside it."""
    from . import score
    score.build()
    return compile_source(SOURCE, _LIB)


def _u16(a):
    return a.ctypes.data_as(_u16p)


def _i32(a):
    return a.ctypes.data_as(_i32p)


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_key.argtypes = [ctypes.c_uint16]
        lib.oracle_key.restype = ctypes.c_uint16
        lib.oracle_is_nan.argtypes = [ctypes.c_uint16]
        lib.oracle_is_nan.restype = ctypes.c_int
        lib.oracle_block_key.argtypes = [_u16p]
        lib.oracle_block_key.restype = ctypes.c_uint16
        lib.oracle_keys.argtypes = [_u16p, ctypes.c_int64, _u16p]
        lib.oracle_keys.restype = None
        lib.oracle_row_keys.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int32, _u16p]
        lib.oracle_row_keys.restype = ctypes.c_int32
        lib.oracle_threshold.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int32,
                                         _u16p, _i32p, _i32p]
        lib.oracle_threshold.restype = ctypes.c_int
        lib.oracle_topk_row.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, _i32p,
                                        ctypes.c_int32, _i32p]
        lib.oracle_topk_row.restype = ctypes.c_int
        lib.oracle_topk_rows.argtypes = [_u16p, ctypes.c_int64, _i32p,
                                         ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _i32p, ctypes.c_int64,
                                         ctypes.c_int32, _i32p]
        lib.oracle_topk_rows.restype = ctypes.c_int
        lib.oracle_topk_rows_ordered.argtypes = [_u16p, ctypes.c_int64, _i32p,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32, _i32p,
                                                 ctypes.c_int64, ctypes.c_int32, _i32p, _i32p,
                                                 _i32p]
        lib.oracle_topk_rows_ordered.restype = ctypes.c_int
        lib.oracle_vector_maxima.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int32, _u16p]
        lib.oracle_vector_maxima.restype = None
        self.lib = lib
        self.path = path

    def key(self, bits):
        """oracle_keys: the order-preserving key of each BF16 pattern."""
        b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
        out = np.empty_like(b)
        self.lib.oracle_keys(_u16(b), b.size, _u16(out))
        return out

    def is_nan(self, bits) -> bool:
        """oracle_is_nan on one pattern."""
        return bool(self.lib.oracle_is_nan(int(bits) & 0xFFFF))

    def block_key(self, x8) -> int:
        """oracle_block_key: key of the NaN-propagating max of 8 patterns."""
        b = np.ascontiguousarray(np.asarray(x8, dtype=np.uint16))
        assert b.size == 8
        return int(self.lib.oracle_block_key(_u16(b)))

    def row_keys(self, row, valid_len: int, mode: int):
        """oracle_row_keys: the element keys of one row (after clamping)."""
        r = np.ascontiguousarray(np.asarray(row, dtype=np.uint16))
        v = max(0, min(int(valid_len), r.size))
        keys = np.empty(max(r.size, 1), dtype=np.uint16)
        n = self.lib.oracle_row_keys(_u16(r), v, mode, _u16(keys))
        return keys[:n].copy()

    def vector_maxima(self, logits, valid_len, width: int | None = None):
        """oracle_vector_maxima per row: the largest key of every 8 logits
        below the row's valid length (0 where none is), [rows, ceil(width/8)]."""
        L = np.ascontiguousarray(np.asarray(logits, dtype=np.uint16))
        if L.ndim == 1:
            L = L[None, :]
        rows = L.shape[0]
        width = L.shape[1] if width is None else int(width)
        vl = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), (rows,))
        nv = (width + 7) // 8
        out = np.zeros((rows, max(nv, 1)), dtype=np.uint16)
        for r in range(rows):
            row = np.ascontiguousarray(L[r])
            self.lib.oracle_vector_maxima(_u16(row), int(vl[r]), width, _u16(out[r]))
        return out[:, :nv]

    def threshold(self, keys, k: int):
        """oracle_threshold: (T, count_gt, count_eq), or None if n <= k."""
        kk = np.ascontiguousarray(np.asarray(keys, dtype=np.uint16))
        if kk.size == 0:
            return None
        T = np.zeros(1, np.uint16)
        gt = np.zeros(1, np.int32)
        eq = np.zeros(1, np.int32)
        rc = self.lib.oracle_threshold(_u16(kk), kk.size, int(k), _u16(T), _i32(gt),
                                       _i32(eq))
        if rc == -1:
            return None
        if rc != 0:
            raise MemoryError("oracle_threshold")
        return int(T[0]), int(gt[0]), int(eq[0])

    def topk_row(self, row, valid_len: int, k: int, mode: int, pages=None,
                 page_size: int = 64):
        """oracle_topk_row on one row (width = len(row))."""
        r = np.ascontiguousarray(np.asarray(row, dtype=np.uint16))
        out = np.empty(k, dtype=np.int32)
        p = None
        if pages is not None:
            p = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
        rc = self.lib.oracle_topk_row(_u16(r), int(valid_len), r.size, int(k), int(mode),
                                      _i32(p) if p is not None else None,
                                      int(page_size), _i32(out))
        if rc != 0:
            raise MemoryError("oracle_topk_row")
        return out

    def topk(self, logits, valid_len, k: int, mode: int, width: int | None = None,
             pages=None, page_size: int = 64, threads: int = 1, rows=None):
        """oracle_topk_rows over a [rows, row_stride] uint16 matrix.

        ``rows`` (optional) restricts the work to the listed row indices; the
        result then has one line per listed row.  ``threads`` > 1 splits the
        rows over that many host threads (ctypes releases the GIL during each
        call).
        """
        L = np.asarray(logits, dtype=np.uint16)
        assert L.ndim == 2
        if rows is not None:
            idx = np.asarray(rows, dtype=np.int64)
            sP = None if pages is None else np.asarray(pages)[idx]
            return self.topk(L[idx], np.asarray(valid_len)[idx], k, mode,
                             width=width if width is not None else L.shape[1],
                             pages=sP, page_size=page_size, threads=threads)
        L = np.ascontiguousarray(L)
        n_rows, stride = L.shape
        if width is None:
            width = stride
        vl = np.ascontiguousarray(np.asarray(valid_len, dtype=np.int32))
        P = None
        pstride = 0
        if pages is not None:
            P = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
            pstride = P.shape[1]
        out = np.empty((n_rows, k), dtype=np.int32)
        pp = _i32(P) if P is not None else None
        lib = self.lib

        def run(b, e):
            rc = lib.oracle_topk_rows(_u16(L), stride, _i32(vl), b, e, int(width),
                                      int(k), int(mode), pp, pstride, int(page_size),
                                      _i32(out))
            if rc != 0:
                raise MemoryError("oracle_topk_rows")

        threads = max(1, min(int(threads), max(n_rows, 1)))
        if threads == 1 or n_rows < 2:
            run(0, n_rows)
        else:
            bounds = np.linspace(0, n_rows, threads + 1).astype(int)
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(lambda i: run(int(bounds[i]), int(bounds[i + 1])),
                            range(threads)))
        return out


    def topk_ordered(self, logits, valid_len, k: int, mode: int, width: int | None = None,
                     pages=None, page_size: int = 64, threads: int = 1):
        """oracle_topk_rows_ordered over a [rows, row_stride] uint16 matrix:
        (out [rows, k], ids [rows, k], valid [rows]), all int32."""
        L = np.ascontiguousarray(np.asarray(logits, dtype=np.uint16))
        assert L.ndim == 2
        n_rows, stride = L.shape
        if width is None:
            width = stride
        vl = np.ascontiguousarray(np.asarray(valid_len, dtype=np.int32))
        P = None
        pstride = 0
        if pages is not None:
            P = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
            pstride = P.shape[1]
        out = np.empty((n_rows, k), dtype=np.int32)
        ids = np.empty((n_rows, k), dtype=np.int32)
        valid = np.empty(n_rows, dtype=np.int32)
        pp = _i32(P) if P is not None else None
        lib = self.lib

        def run(b, e):
            rc = lib.oracle_topk_rows_ordered(_u16(L), stride, _i32(vl), b, e, int(width),
                                              int(k), int(mode), pp, pstride, int(page_size),
                                              _i32(out), _i32(ids), _i32(valid))
            if rc != 0:
                raise MemoryError("oracle_topk_rows_ordered")

        threads = max(1, min(int(threads), max(n_rows, 1)))
        if threads == 1 or n_rows < 2:
            run(0, n_rows)
        else:
            bounds = np.linspace(0, n_rows, threads + 1).astype(int)
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(lambda i: run(int(bounds[i]), int(bounds[i + 1])),
                            range(threads)))
        return out, ids, valid

def vector_maxima(logits, valid_len, width=None):
    """oracle_vector_maxima per row: uint16 [rows, ceil(width / 8)]."""
    return default().vector_maxima(logits, valid_len, width)


def default() -> Oracle:
    """The oracle built from oracle/topk_oracle.c (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            if (not os.path.exists(_LIB)
                    or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE)):
                build()
            _default = Oracle(_LIB)
        return _default


def key(bits):
    return default().key(bits)


def is_nan(bits):
    return default().is_nan(bits)


def block_key(x8):
    return default().block_key(x8)


def row_keys(row, valid_len, mode):
    return default().row_keys(row, valid_len, mode)


def threshold(keys, k):
    return default().threshold(keys, k)


def topk_row(row, valid_len, k, mode, pages=None, page_size=64):
    return default().topk_row(row, valid_len, k, mode, pages, page_size)


def topk(logits, valid_len, k, mode, width=None, pages=None, page_size=64, threads=1,
         rows=None):
    return default().topk(logits, valid_len, k, mode, width=width, pages=pages,
                          page_size=page_size, threads=threads, rows=rows)


def topk_ordered(logits, valid_len, k, mode, width=None, pages=None, page_size=64, threads=1):
    return default().topk_ordered(logits, valid_len, k, mode, width=width, pages=pages,
                                  page_size=page_size, threads=threads)
