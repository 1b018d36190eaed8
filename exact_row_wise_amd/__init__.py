"""exact_row_wise_amd -- exact per-row top-k of BF16 logits on MI355X.

The work is done by ``libtopk.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/libtopk.h``).  This package only marshals torch
tensors (device memory, streams) into that C call; there is no other
implementation and no fallback: if the library is missing the call raises.
"""
from ._binding import (  # noqa: F401
    MODE_BLOCK,
    MODE_TOKEN,
    PATH_DIRECT_FORCED,
    PATH_DIRECT_MISJUDGED,
    PATH_DIRECT_OVERFLOW,
    PATH_SAMPLED,
    PATH_SAMPLED_TIES,
    PATH_DIRECT_DENSE,
    PATH_SHORT,
    PATH_TOPS,
    TopkError,
    fp8_mqa_logits,
    mxfp4_mqa_logits,
    library,
    probe_library,
    stream_read,
    topk_bf16_rows_noalloc,
    topk_bf16_rows_ordered,
    library_path,
    release_scratch,
    reserve_scratch,
    status_string,
    topk_bf16_rows,
    topk_bf16_rows_tops,
    vector_maxima,
)
