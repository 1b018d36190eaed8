"""ctypes wrapper of ``score_oracle.c`` (test infrastructure only): the FP8
and MXFP4 MQA indexer logits at the precision the K3.1 indexer page states.

Each method names the C function it calls; the C source cites the passages
it follows.  ``ScoreOracle(path)`` wraps one compiled copy, so that tests can
also load a copy built from a deliberately altered source.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from .oracle import compile_source

HEADS = 32
DIM = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "score_oracle.c")
_LIB = os.path.join(_HERE, "libscore_oracle.so")
_lock = threading.Lock()
_default = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)


def build() -> str:
    """Compile oracle/score_oracle.c into oracle/libscore_oracle.so (-lm)."""
    return compile_source(SOURCE, _LIB, libs=("-lm",))


class ScoreOracle:
    """One loaded copy of the scorer oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3.restype = ctypes.c_longdouble
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_longdouble
        lib.oracle_bf16_round.argtypes = [ctypes.c_longdouble]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_mqa_logit.argtypes = [_u8p, _u16p, _u8p, ctypes.c_uint8, ctypes.c_double,
                                         _u16p, _u16p, _u16p]
        lib.oracle_mqa_logit.restype = None
        lib.oracle_mqa_logits.argtypes = [_u8p, _u16p, ctypes.c_int32, _u8p, _u8p,
                                          ctypes.c_int32, ctypes.c_double, _u16p, _u16p, _u16p]
        lib.oracle_mqa_logits.restype = None
        lib.oracle_e2m1.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1.restype = ctypes.c_longdouble
        lib.oracle_mxfp4_logit.argtypes = [_u8p, _u8p, _u16p, _u8p, _u8p, ctypes.c_double,
                                           _u16p, _u16p, _u16p]
        lib.oracle_mxfp4_logit.restype = None
        lib.oracle_mxfp4_logits.argtypes = [_u8p, _u8p, _u16p, ctypes.c_int32, _u8p, _u8p,
                                            ctypes.c_int32, ctypes.c_double, _u16p, _u16p, _u16p]
        lib.oracle_mxfp4_logits.restype = None
        self.lib = lib
        self.path = path

    def e4m3(self, codes):
        """oracle_e4m3 of each byte (float64 of the exact value; NaN for NaN)."""
        c = np.asarray(codes, dtype=np.uint8).ravel()
        return np.array([float(self.lib.oracle_e4m3(int(x))) for x in c]).reshape(np.shape(codes))

    def bf16_value(self, bits):
        """oracle_bf16_value of each pattern (float64)."""
        b = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([float(self.lib.oracle_bf16_value(int(x))) for x in b]).reshape(np.shape(bits))

    def bf16_round(self, values):
        """oracle_bf16_round of each value (given as float64)."""
        v = np.asarray(values, dtype=np.float64).ravel()
        return np.array([self.lib.oracle_bf16_round(float(x)) for x in v],
                        dtype=np.uint16).reshape(np.shape(values))

    def mqa_logits(self, q, w, keys, scales, delta: float = 0.0):
        """oracle_mqa_logits for one request: q uint8 [rows, HEADS, DIM], w
        BF16 patterns [rows, HEADS], keys uint8 [nkeys, DIM], scales uint8
        [nkeys].  Returns (exact, lo, hi), uint16 [rows, nkeys] each."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        keys = np.ascontiguousarray(keys, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        rows, nk = q.shape[0], keys.shape[0]
        assert q.shape[1:] == (HEADS, DIM) and w.shape == (rows, HEADS)
        assert keys.shape[1] == DIM and scales.shape == (nk,)
        ex = np.empty((rows, nk), np.uint16)
        lo = np.empty_like(ex)
        hi = np.empty_like(ex)
        if rows and nk:
            self.lib.oracle_mqa_logits(q.ctypes.data_as(_u8p), w.ctypes.data_as(_u16p), rows,
                                       keys.ctypes.data_as(_u8p), scales.ctypes.data_as(_u8p),
                                       nk, float(delta), ex.ctypes.data_as(_u16p),
                                       lo.ctypes.data_as(_u16p), hi.ctypes.data_as(_u16p))
        return ex, lo, hi

    def mqa_logit(self, q, w, key, scale: int, delta: float = 0.0):
        """oracle_mqa_logit: (exact, lo, hi) patterns of one query row and key."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        key = np.ascontiguousarray(key, dtype=np.uint8)
        ex, lo, hi = ctypes.c_uint16(), ctypes.c_uint16(), ctypes.c_uint16()
        self.lib.oracle_mqa_logit(q.ctypes.data_as(_u8p), w.ctypes.data_as(_u16p),
                                  key.ctypes.data_as(_u8p), int(scale), float(delta),
                                  ctypes.byref(ex), ctypes.byref(lo), ctypes.byref(hi))
        return int(ex.value), int(lo.value), int(hi.value)


    def e2m1(self, nibbles):
        """oracle_e2m1 of each 4-bit code (float64 of the exact value)."""
        c = np.asarray(nibbles, dtype=np.uint8).ravel()
        return np.array([float(self.lib.oracle_e2m1(int(x))) for x in c]).reshape(np.shape(nibbles))

    def mxfp4_logits(self, q, q_scale, w, keys, key_scales, delta: float = 0.0):
        """oracle_mxfp4_logits for one request: q uint8 [rows, HEADS, DIM / 2]
        (E2M1, low nibble first), q_scale uint8 [rows, HEADS, 4], w BF16
        patterns [rows, HEADS], keys uint8 [nkeys, DIM / 2], key_scales uint8
        [nkeys, 4].  Returns (exact, lo, hi), uint16 [rows, nkeys] each."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        qs = np.ascontiguousarray(q_scale, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        keys = np.ascontiguousarray(keys, dtype=np.uint8)
        ks = np.ascontiguousarray(key_scales, dtype=np.uint8)
        rows, nk = q.shape[0], keys.shape[0]
        assert q.shape[1:] == (HEADS, DIM // 2) and qs.shape == (rows, HEADS, 4)
        assert w.shape == (rows, HEADS) and keys.shape[1] == DIM // 2 and ks.shape == (nk, 4)
        ex = np.empty((rows, nk), np.uint16)
        lo = np.empty_like(ex)
        hi = np.empty_like(ex)
        if rows and nk:
            self.lib.oracle_mxfp4_logits(q.ctypes.data_as(_u8p), qs.ctypes.data_as(_u8p),
                                         w.ctypes.data_as(_u16p), rows,
                                         keys.ctypes.data_as(_u8p), ks.ctypes.data_as(_u8p), nk,
                                         float(delta), ex.ctypes.data_as(_u16p),
                                         lo.ctypes.data_as(_u16p), hi.ctypes.data_as(_u16p))
        return ex, lo, hi

    def mxfp4_logit(self, q, q_scale, w, key, key_scale, delta: float = 0.0):
        """oracle_mxfp4_logit: (exact, lo, hi) patterns of one query row and key."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        qs = np.ascontiguousarray(q_scale, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        key = np.ascontiguousarray(key, dtype=np.uint8)
        ks = np.ascontiguousarray(key_scale, dtype=np.uint8)
        ex, lo, hi = ctypes.c_uint16(), ctypes.c_uint16(), ctypes.c_uint16()
        self.lib.oracle_mxfp4_logit(q.ctypes.data_as(_u8p), qs.ctypes.data_as(_u8p),
                                    w.ctypes.data_as(_u16p), key.ctypes.data_as(_u8p),
                                    ks.ctypes.data_as(_u8p), float(delta), ctypes.byref(ex),
                                    ctypes.byref(lo), ctypes.byref(hi))
        return int(ex.value), int(lo.value), int(hi.value)


def load() -> ScoreOracle:
    """The scorer oracle built from oracle/score_oracle.c (built on first use)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
                build()
            _default = ScoreOracle(_LIB)
        return _default
