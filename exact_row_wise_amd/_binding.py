"""ctypes binding of libtopk (argument marshalling only).

``topk_bf16_rows`` mirrors the C entry point of the same name in
``include/libtopk.h``: it checks that the tensors are on the GPU with the
right dtype and layout, passes their device pointers, sizes and the
current HIP stream, and raises on a non-zero status.  Every step of the
selection runs in the HIP kernels of libtopk.so.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # loaded first: libtopk then shares torch's HIP runtime

MODE_TOKEN = 0
MODE_BLOCK = 1

PATH_SHORT = 0
PATH_SAMPLED = 1
PATH_SAMPLED_TIES = 2
PATH_DIRECT_FORCED = 3
PATH_DIRECT_MISJUDGED = 4
PATH_DIRECT_OVERFLOW = 5
PATH_TOPS = 6
PATH_DIRECT_DENSE = 7

ERR_UNSUPPORTED = -4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libtopk.so")
_PROBE_LIB = os.path.join(_HERE, "libtopk_probe.so")
_lock = threading.Lock()
_lib = None
_probe = None


class TopkError(RuntimeError):
    """A non-zero status from libtopk."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"libtopk status {status}: {detail}")
        self.status = status


class _BlockTable(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
                ("page_size", ctypes.c_int32)]


class _Options(ctypes.Structure):
    _fields_ = [("force_direct", ctypes.c_int32), ("path_codes", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB


def library():
    """Load libtopk.so (built in-tree by ``python -m exact_row_wise_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            raise ImportError(
                f"{_LIB} is missing: build it with `python -m exact_row_wise_amd.build`")
        lib = ctypes.CDLL(_LIB)
        sig = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_BlockTable),
               ctypes.c_void_p]
        lib.topk_bf16_rows.argtypes = sig + [ctypes.c_void_p]
        lib.topk_bf16_rows.restype = ctypes.c_int
        lib.topk_bf16_rows_ex.argtypes = sig + [ctypes.POINTER(_Options), ctypes.c_void_p]
        lib.topk_bf16_rows_ex.restype = ctypes.c_int
        lib.topk_bf16_rows_noalloc.argtypes = sig + [ctypes.c_void_p]
        lib.topk_bf16_rows_noalloc.restype = ctypes.c_int
        osig = sig + [ctypes.c_void_p, ctypes.c_void_p]
        lib.topk_bf16_rows_ordered.argtypes = osig + [ctypes.c_void_p]
        lib.topk_bf16_rows_ordered.restype = ctypes.c_int
        lib.topk_bf16_rows_ordered_ex.argtypes = osig + [ctypes.POINTER(_Options),
                                                         ctypes.c_void_p]
        lib.topk_bf16_rows_ordered_ex.restype = ctypes.c_int
        lib.topk_bf16_rows_tops.argtypes = sig[:7] + [ctypes.c_void_p, ctypes.c_int64] + sig[7:] + [
            ctypes.POINTER(_Options), ctypes.c_void_p]
        lib.topk_bf16_rows_tops.restype = ctypes.c_int
        lib.topk_bf16_vector_maxima.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_void_p]
        lib.topk_bf16_vector_maxima.restype = ctypes.c_int
        lib.topk_fp8_mqa_logits.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64,
                                            ctypes.c_void_p] + [ctypes.c_int32] * 3 + [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.topk_fp8_mqa_logits.restype = ctypes.c_int
        lib.topk_mxfp4_mqa_logits.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64,
                                              ctypes.c_void_p] + [ctypes.c_int32] * 3 + [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.topk_mxfp4_mqa_logits.restype = ctypes.c_int
        lib.topk_status_string.argtypes = [ctypes.c_int]
        lib.topk_status_string.restype = ctypes.c_char_p
        lib.topk_last_error.argtypes = []
        lib.topk_last_error.restype = ctypes.c_char_p
        lib.topk_reserve_scratch.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p]
        lib.topk_reserve_scratch.restype = ctypes.c_int
        lib.topk_release_scratch.argtypes = []
        lib.topk_release_scratch.restype = ctypes.c_int
        _lib = lib
        return lib


def probe_library():
    """Load libtopk_probe.so (the streaming-read probe, built beside libtopk)."""
    global _probe
    with _lock:
        if _probe is not None:
            return _probe
        if not os.path.exists(_PROBE_LIB):
            raise ImportError(f"{_PROBE_LIB} is missing: build it with "
                              "`python -m exact_row_wise_amd.build`")
        lib = ctypes.CDLL(_PROBE_LIB)
        lib.topk_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                               ctypes.c_void_p]
        lib.topk_probe_stream_read.restype = ctypes.c_int
        _probe = lib
        return lib


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream: torch.cuda.Stream | None = None):
    """topk_probe_stream_read over all of `buf` (a contiguous GPU tensor whose
    byte size is a multiple of 16, zero-filled); `sink` holds 256 int32."""
    if not buf.is_contiguous() or buf.device.type != "cuda" or sink.numel() < 256:
        raise ValueError("stream_read needs a contiguous GPU buffer and a 256-word sink")
    nbytes = buf.numel() * buf.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    rc = probe_library().topk_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(),
                                                ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise TopkError(rc, "topk_probe_stream_read failed")


def status_string(status: int) -> str:
    return library().topk_status_string(int(status)).decode()


def reserve_scratch(rows: int, width: int, k: int, mode=MODE_TOKEN, ordered: bool = False,
                    stream: torch.cuda.Stream | None = None) -> None:
    """topk_reserve_scratch (include/libtopk.h): set up and pin the scratch of
    `stream` (default: the current stream) for calls of up to `rows` rows of
    this width, k and mode, before capturing such calls into a graph."""
    lib = library()
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = lib.topk_reserve_scratch(int(rows), int(width), int(k), _mode(mode),
                                  1 if ordered else 0, ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise TopkError(rc, lib.topk_last_error().decode())


def release_scratch() -> None:
    rc = library().topk_release_scratch()
    if rc != 0:
        raise TopkError(rc, library().topk_last_error().decode())


def _mode(mode) -> int:
    if mode in (MODE_TOKEN, "token"):
        return MODE_TOKEN
    if mode in (MODE_BLOCK, "block"):
        return MODE_BLOCK
    return int(mode)  # passed through; the library rejects unknown modes


def topk_bf16_rows(logits: torch.Tensor, valid_len: torch.Tensor, k: int, mode=MODE_TOKEN,
                   block_table: torch.Tensor | None = None, page_size: int = 64,
                   out: torch.Tensor | None = None, width: int | None = None,
                   force_direct: bool = False, path_codes: torch.Tensor | None = None,
                   stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Exact top-k indices of every row (see include/libtopk.h).

    logits      [rows, >= width] BF16 (or int16/uint16 bit patterns) on the
                GPU; unit stride along a row, the row stride a multiple of 8
                elements, 16-byte aligned
    valid_len   int32 [rows] on the GPU
    k           1 .. 2048
    mode        "token"/0 or "block"/1
    block_table optional int32 [rows, >= ceil(width / page_size)] on the GPU
    out         optional int32 [rows, k] contiguous on the GPU (allocated if None)
    width       logits per row (default: logits.shape[1])
    force_direct, path_codes   test hooks of topk_bf16_rows_ex
    stream      torch stream (default: the current stream)
    Returns out.
    """
    return _call(logits, valid_len, k, mode, block_table, page_size, out, width, force_direct,
                 path_codes, stream)[0]


def topk_bf16_rows_noalloc(logits: torch.Tensor, valid_len: torch.Tensor, k: int,
                           mode=MODE_TOKEN, block_table: torch.Tensor | None = None,
                           page_size: int = 64, out: torch.Tensor | None = None,
                           width: int | None = None,
                           stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """topk_bf16_rows through the entry point that allocates nothing (see
    include/libtopk.h): `out` must be given, and the library uses its fixed
    per-device scratch (calls overlapping on one GPU race).  Returns out."""
    if out is None:
        raise ValueError("topk_bf16_rows_noalloc needs a preallocated out")
    return _call(logits, valid_len, k, mode, block_table, page_size, out, width, False, None,
                 stream, noalloc=True)[0]


def topk_bf16_rows_tops(logits: torch.Tensor, valid_len: torch.Tensor, k: int, tops: torch.Tensor,
                        mode=MODE_TOKEN, block_table: torch.Tensor | None = None,
                        page_size: int = 64, out: torch.Tensor | None = None,
                        width: int | None = None, force_direct: bool = False,
                        path_codes: torch.Tensor | None = None,
                        stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """topk_bf16_rows given the rows' vector maxima (see include/libtopk.h):
    tops is [rows, >= ceil(width / 8)] 16-bit (int16/uint16) on the GPU, unit
    stride along a row, the row stride a multiple of 8, 16-byte aligned, each
    entry the largest key of its 8 logits below the valid length (0 where
    none is), as vector_maxima writes it.  Other arguments as for
    topk_bf16_rows.  Returns out."""
    return _call(logits, valid_len, k, mode, block_table, page_size, out, width, force_direct,
                 path_codes, stream, tops=tops)[0]


def vector_maxima(logits: torch.Tensor, valid_len: torch.Tensor, width: int | None = None,
                  tops: torch.Tensor | None = None,
                  stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """The side array topk_bf16_rows_tops reads (topk_bf16_vector_maxima in
    include/libtopk.h): tops[r, j] = the largest key among logits 8j .. 8j+7
    of row r below valid_len[r], 0 where none is.  tops (int16 [rows,
    >= ceil(width / 8) rounded up to 8], unit stride along a row, row stride a
    multiple of 8) is allocated if None.  Returns tops."""
    lib = library()
    if logits.dim() != 2 or logits.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("logits must be 2-D 16-bit [rows, row_stride]")
    rows = logits.shape[0]
    if width is None:
        width = logits.shape[1]
    if int(width) < 0 or int(width) > logits.shape[1]:
        raise ValueError(f"width {width} outside [0, logits.shape[1] = {logits.shape[1]}]")
    if logits.shape[1] > 1 and logits.stride(1) != 1:
        raise ValueError("logits rows must have unit stride")
    dev = logits.device
    if valid_len.dtype != torch.int32 or valid_len.numel() != rows or valid_len.device != dev:
        raise ValueError("valid_len must be int32 [rows] on the same GPU")
    valid_len = valid_len.contiguous()
    nv = -(-int(width) // 8)
    if tops is None:
        tops = torch.zeros((rows, max(8, -(-nv // 8) * 8)), dtype=torch.int16, device=dev)
    elif (tops.dtype not in (torch.int16, torch.uint16) or tops.dim() != 2
          or tops.shape[0] != rows or tops.shape[1] < nv or tops.device != dev
          or (rows > 0 and tops.shape[1] > 1 and tops.stride(1) != 1)):
        raise ValueError("tops must be 16-bit [rows, >= ceil(width / 8)] on the same GPU")
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rc = lib.topk_bf16_vector_maxima(logits.data_ptr(), int(logits.stride(0)),
                                         valid_len.data_ptr(), int(rows), int(width),
                                         tops.data_ptr(), int(tops.stride(0)),
                                         ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise TopkError(rc, lib.topk_last_error().decode())
    return tops


def fp8_mqa_logits(q: torch.Tensor, w: torch.Tensor, keys: torch.Tensor,
                   key_scale: torch.Tensor, valid_len: torch.Tensor, qpr: int = 1,
                   width: int | None = None, logits: torch.Tensor | None = None,
                   tops: torch.Tensor | None = None,
                   stream: torch.cuda.Stream | None = None):
    """The FP8 MQA indexer logits and their vector maxima
    (topk_fp8_mqa_logits in include/libtopk.h).
    q          uint8 [rows, 32, 128] (E4M3 bytes), contiguous
    w          BF16 or 16-bit patterns [rows, 32], contiguous
    keys       uint8 [requests, key_stride, 128] (E4M3 bytes), contiguous
    key_scale  uint8 [requests, key_stride] (UE8M0 bytes)
    valid_len  int32 [rows]; rows = requests * qpr
    logits     16-bit [rows, >= width] (unit stride along a row), tops 16-bit
               [rows, >= ceil(width / 8) rounded up to 8]; allocated if None
    Returns (logits, tops)."""
    return _score(False, q, None, w, keys, key_scale, valid_len, qpr, width, logits, tops,
                  stream)


def mxfp4_mqa_logits(q: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor,
                     keys: torch.Tensor, key_scale: torch.Tensor, valid_len: torch.Tensor,
                     qpr: int = 1, width: int | None = None, logits: torch.Tensor | None = None,
                     tops: torch.Tensor | None = None,
                     stream: torch.cuda.Stream | None = None):
    """The MXFP4 MQA indexer logits and their vector maxima
    (topk_mxfp4_mqa_logits in include/libtopk.h).
    q          uint8 [rows, 32, 64] (E2M1, two a byte, low nibble first)
    q_scale    uint8 [rows, 32, 4] (UE8M0 of each head's 32-dim blocks)
    keys       uint8 [requests, key_stride, 64] (E2M1)
    key_scale  uint8 [requests, key_stride, 4] (UE8M0 of each key's blocks)
    the rest as for fp8_mqa_logits.  Returns (logits, tops)."""
    return _score(True, q, q_scale, w, keys, key_scale, valid_len, qpr, width, logits, tops,
                  stream)


def _score(fp4, q, q_scale, w, keys, key_scale, valid_len, qpr, width, logits, tops, stream):
    lib = library()
    qb = 64 if fp4 else 128
    if q.dtype != torch.uint8 or q.dim() != 3 or tuple(q.shape[1:]) != (32, qb) or not q.is_contiguous():
        raise ValueError(f"q must be contiguous uint8 [rows, 32, {qb}]")
    rows = q.shape[0]
    dev = q.device
    if fp4 and (q_scale is None or q_scale.dtype != torch.uint8
                or tuple(q_scale.shape) != (rows, 32, 4) or not q_scale.is_contiguous()
                or q_scale.device != dev):
        raise ValueError("q_scale must be contiguous uint8 [rows, 32, 4] on the same GPU")
    if w.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or tuple(w.shape) != (rows, 32) \
            or not w.is_contiguous() or w.device != dev:
        raise ValueError("w must be contiguous 16-bit [rows, 32] on the same GPU")
    if keys.dtype != torch.uint8 or keys.dim() != 3 or keys.shape[2] != qb \
            or not keys.is_contiguous() or keys.device != dev:
        raise ValueError(f"keys must be contiguous uint8 [requests, key_stride, {qb}]")
    requests, key_stride = keys.shape[0], keys.shape[1]
    ks_shape = (requests, key_stride, 4) if fp4 else (requests, key_stride)
    if key_scale.dtype != torch.uint8 or tuple(key_scale.shape) != ks_shape \
            or not key_scale.is_contiguous() or key_scale.device != dev:
        raise ValueError(f"key_scale must be contiguous uint8 {list(ks_shape)}")
    if int(qpr) < 1 or rows != requests * int(qpr):
        raise ValueError(f"rows {rows} must be requests {requests} x qpr {qpr}")
    if valid_len.dtype != torch.int32 or valid_len.numel() != rows or valid_len.device != dev:
        raise ValueError("valid_len must be int32 [rows] on the same GPU")
    valid_len = valid_len.contiguous()
    if width is None:
        width = key_stride
    nv = -(-int(width) // 8)
    if logits is None:
        logits = torch.zeros((rows, max(8, -(-int(width) // 8) * 8)), dtype=torch.int16, device=dev)
    elif (logits.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or logits.dim() != 2
          or logits.shape[0] != rows or logits.shape[1] < int(width) or logits.device != dev
          or (logits.shape[1] > 1 and logits.stride(1) != 1)):
        raise ValueError("logits must be 16-bit [rows, >= width] on the same GPU")
    if tops is None:
        tops = torch.zeros((rows, max(8, -(-nv // 8) * 8)), dtype=torch.int16, device=dev)
    elif (tops.dtype not in (torch.int16, torch.uint16) or tops.dim() != 2
          or tops.shape[0] != rows or tops.shape[1] < nv or tops.device != dev
          or (tops.shape[1] > 1 and tops.stride(1) != 1)):
        raise ValueError("tops must be 16-bit [rows, >= ceil(width / 8)] on the same GPU")
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        tail = (int(key_stride), valid_len.data_ptr(), int(rows), int(qpr), int(width),
                logits.data_ptr(), int(logits.stride(0)), tops.data_ptr(), int(tops.stride(0)),
                ctypes.c_void_p(s.cuda_stream))
        if fp4:
            rc = lib.topk_mxfp4_mqa_logits(q.data_ptr(), q_scale.data_ptr(), w.data_ptr(),
                                           keys.data_ptr(), key_scale.data_ptr(), *tail)
        else:
            rc = lib.topk_fp8_mqa_logits(q.data_ptr(), w.data_ptr(), keys.data_ptr(),
                                         key_scale.data_ptr(), *tail)
    if rc != 0:
        raise TopkError(rc, lib.topk_last_error().decode())
    return logits, tops


def topk_bf16_rows_ordered(logits: torch.Tensor, valid_len: torch.Tensor, k: int,
                           mode=MODE_TOKEN, block_table: torch.Tensor | None = None,
                           page_size: int = 64, out: torch.Tensor | None = None,
                           valid: torch.Tensor | None = None, ids: torch.Tensor | None = None,
                           want_ids: bool = True, width: int | None = None,
                           force_direct: bool = False, path_codes: torch.Tensor | None = None,
                           stream: torch.cuda.Stream | None = None):
    """Deterministic ordered top-k of every row (see include/libtopk.h):
    the selected indices in ascending order, ties at the k-th key from the
    lowest indices, -1 past the count.  Arguments as for topk_bf16_rows, plus
    valid (int32 [rows]) and ids (int32 [rows, k]), allocated if None (ids
    only when want_ids).  Returns (out, valid, ids or None)."""
    return _call(logits, valid_len, k, mode, block_table, page_size, out, width, force_direct,
                 path_codes, stream, True, valid, ids, want_ids)


def _call(logits, valid_len, k, mode, block_table, page_size, out, width, force_direct,
          path_codes, stream, ordered=False, valid=None, ids=None, want_ids=False,
          noalloc=False, tops=None):
    lib = library()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, row_stride]")
    if logits.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("logits must be bfloat16 (or 16-bit integer bit patterns)")
    rows = logits.shape[0]
    if width is None:
        width = logits.shape[1]
    if int(width) < 0 or int(width) > logits.shape[1]:
        raise ValueError(f"width {width} outside [0, logits.shape[1] = {logits.shape[1]}]")
    if logits.shape[1] > 1 and logits.stride(1) != 1:
        raise ValueError("logits rows must have unit stride")
    row_stride = logits.stride(0)
    if valid_len.dtype != torch.int32 or valid_len.numel() != rows:
        raise ValueError("valid_len must be int32 [rows]")
    dev = logits.device
    if dev.type != "cuda" or valid_len.device != dev:
        raise ValueError("logits and valid_len must be on the same GPU")
    valid_len = valid_len.contiguous()
    if out is None:
        out = torch.empty((rows, int(k)), dtype=torch.int32, device=dev)
    elif (out.dtype != torch.int32 or tuple(out.shape) != (rows, int(k))
          or not out.is_contiguous() or out.device != dev):
        raise ValueError("out must be a contiguous int32 [rows, k] tensor on the same GPU")
    if ordered:
        if valid is None:
            valid = torch.empty(rows, dtype=torch.int32, device=dev)
        elif (valid.dtype != torch.int32 or valid.numel() != rows or not valid.is_contiguous()
              or valid.device != dev):
            raise ValueError("valid must be a contiguous int32 [rows] tensor on the same GPU")
        if ids is None and want_ids:
            ids = torch.empty((rows, int(k)), dtype=torch.int32, device=dev)
        elif ids is not None and (ids.dtype != torch.int32 or tuple(ids.shape) != (rows, int(k))
                                  or not ids.is_contiguous() or ids.device != dev):
            raise ValueError("ids must be a contiguous int32 [rows, k] tensor on the same GPU")
    bt = None
    if block_table is not None:
        if (block_table.dtype != torch.int32 or block_table.dim() != 2
                or block_table.device != dev or block_table.shape[0] != rows
                or (rows > 0 and block_table.stride(1) != 1)):
            raise ValueError("block_table must be int32 [rows, pages] on the same GPU")
        if int(page_size) >= 1 and block_table.shape[1] < -(-int(width) // int(page_size)):
            raise ValueError(f"block_table rows hold {block_table.shape[1]} pages; width "
                             f"{width} needs ceil(width / page_size) of them")
        bt = _BlockTable(block_table.data_ptr(), block_table.stride(0), int(page_size))
    if tops is not None:
        if (tops.dtype not in (torch.int16, torch.uint16) or tops.dim() != 2
                or tops.shape[0] != rows or tops.device != dev
                or (rows > 0 and tops.shape[1] > 1 and tops.stride(1) != 1)):
            raise ValueError("tops must be 16-bit [rows, >= ceil(width / 8)] on the same GPU")
        if tops.shape[1] < -(-int(width) // 8):
            raise ValueError(f"tops rows hold {tops.shape[1]} maxima; width {width} needs "
                             f"ceil(width / 8) of them")
    opts = None
    if force_direct or path_codes is not None:
        if path_codes is not None and (path_codes.dtype != torch.int32
                                       or path_codes.numel() != rows
                                       or path_codes.device != dev):
            raise ValueError("path_codes must be int32 [rows] on the same GPU")
        opts = _Options(1 if force_direct else 0,
                        path_codes.data_ptr() if path_codes is not None else None)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        args = (logits.data_ptr(), int(row_stride), valid_len.data_ptr(), int(rows),
                int(width), int(k), _mode(mode), ctypes.byref(bt) if bt is not None else None,
                out.data_ptr())
        st = ctypes.c_void_p(s.cuda_stream)
        if ordered:
            args += (valid.data_ptr(), ids.data_ptr() if ids is not None else None)
            if opts is None:
                rc = lib.topk_bf16_rows_ordered(*args, st)
            else:
                rc = lib.topk_bf16_rows_ordered_ex(*args, ctypes.byref(opts), st)
        elif noalloc:
            rc = lib.topk_bf16_rows_noalloc(*args, st)
        elif tops is not None:
            targs = args[:7] + (tops.data_ptr(), int(tops.stride(0))) + args[7:]
            rc = lib.topk_bf16_rows_tops(*targs, ctypes.byref(opts) if opts is not None else None,
                                         st)
        elif opts is None:
            rc = lib.topk_bf16_rows(*args, st)
        else:
            rc = lib.topk_bf16_rows_ex(*args, ctypes.byref(opts), st)
    if rc != 0:
        raise TopkError(rc, lib.topk_last_error().decode())
    return out, valid, ids
