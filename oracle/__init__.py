"""CPU oracle for exact per-row BF16 top-k (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product library
(``exact_row_wise_amd``) never imports it and shares no code with it.

The arithmetic lives in ``topk_oracle.c`` (plain C: per row, element keys,
a full ``qsort`` by (key desc, index asc), the first k; the ordered result
sorts those k by index; the side array of vector maxima is a plain loop),
and in ``score_oracle.c`` (the FP8 MQA indexer logits: exact dot products,
BF16 roundings in the stated order; ``score.py`` wraps it).  This package
only compiles them with gcc and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    MODE_TOKEN,
    MODE_BLOCK,
    SOURCE,
    Oracle,
    build,
    compile_source,
    default,
    key,
    is_nan,
    block_key,
    row_keys,
    threshold,
    topk_row,
    topk,
    topk_ordered,
    vector_maxima,
    lib_path,
)
from . import score  # noqa: F401
