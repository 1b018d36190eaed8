"""The CPU oracle against its pins, and the pins against planted mistakes.

A planted mistake is a one-line change to a temporary copy of
oracle/topk_oracle.c, compiled on the CPU; the real oracle is untouched.
Every such copy must fail at least one pin.
"""
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (description, exact text in topk_oracle.c, replacement)
MUTANTS = [
    ("negative key flips 15 bits", "return (uint16_t)(bits ^ 0xFFFFu);",
     "return (uint16_t)(bits ^ 0x7FFFu);"),
    ("positive key not flipped", "return (uint16_t)(bits ^ 0x8000u);",
     "return (uint16_t)(bits);"),
    ("sign test inverted", "if (bits & 0x8000u)\n        return (uint16_t)(bits ^ 0xFFFFu);",
     "if (!(bits & 0x8000u))\n        return (uint16_t)(bits ^ 0xFFFFu);"),
    ("ascending sort", "return a->key > b->key ? -1 : 1;", "return a->key > b->key ? 1 : -1;"),
    ("newest block not pinned", "keys[n - 1] = oracle_key(0x7F80u);",
     "keys[n - 1] = oracle_block_key(row + (int64_t)8 * (n - 1));"),
    ("-inf blocks keep their index", "out[j] = -1;\n    for (j = cnt",
     "out[j] = out[j];\n    for (j = cnt"),
    ("block count floors", "return (v + 7) / 8;", "return v / 8;"),
    ("page offset dropped", "* page_size + out[j] % page_size;", "* page_size;"),
    ("page index by offset", "pages[out[j] / page_size]", "pages[out[j] % page_size]"),
    ("NaN ignored in block max", "return oracle_key(0x7FFFu);", "break;"),
    ("inf counted as NaN", "((bits & 0x007Fu) != 0u)", "1"),
    ("no upper clamp", "if (v > width)\n        return width;", "if (v > width)\n        return v - 0;"),
    ("k-th is one off", "t = items[k - 1].key;", "t = items[k].key;"),
    ("short rows use <", "if (n <= k) {\n        for (j = 0; j < n; ++j)\n            out[j] = j;",
     "if (n < k) {\n        for (j = 0; j < n; ++j)\n            out[j] = j;"),
    ("block max keeps first", "if (k > best)\n            best = k;", "if (k < best)\n            best = k;"),
    ("tie count includes >", "else if (keys[i] == t)", "if (keys[i] >= t)"),
    ("ordered: no index sort", "qsort(sel, (size_t)cnt, sizeof(int32_t), by_index_asc);", ";"),
    ("ordered: descending index", "return a < b ? -1 : (a > b ? 1 : 0);",
     "return a < b ? 1 : (a > b ? -1 : 0);"),
    ("ordered: count is k", "*valid = cnt;", "*valid = k;"),
    ("ordered: ids mapped", "ids[j] = i;", "ids[j] = o;"),
    ("rows: table row by page size",
     "const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;\n        int rc = oracle_topk_row(",
     "const int32_t *prow = pages ? pages + (int64_t)r * page_size : NULL;\n        int rc = oracle_topk_row("),
    ("rows: logits row by width", "oracle_topk_row(logits + (int64_t)r * row_stride,",
     "oracle_topk_row(logits + (int64_t)r * width,"),
    ("maxima ignore the length", "i < 8 * j + 8 && i < v;", "i < 8 * j + 8 && i < width;"),
    ("maxima keep the smallest", "            if (k > best)\n                best = k;",
     "            if (k < best || i == 8 * j)\n                best = k;"),
    ("maxima of raw bits", "uint16_t k = oracle_key(row[i]);", "uint16_t k = row[i];"),
    ("maxima one logit apart", "for (i = 8 * j; i < 8 * j + 8", "for (i = 8 * j + 1; i < 8 * j + 8"),
    ("rows: output row by width", "out + (int64_t)r * k);", "out + (int64_t)r * width);"),
    ("rows: first row skipped", "for (r = row_begin; r < row_end; ++r) {\n        const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;\n        int rc = oracle_topk_row(",
     "for (r = row_begin + 1; r < row_end; ++r) {\n        const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;\n        int rc = oracle_topk_row("),
    ("ordered rows: table row by page size",
     "const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;\n        int rc = oracle_topk_row_ordered(",
     "const int32_t *prow = pages ? pages + (int64_t)r * page_size : NULL;\n        int rc = oracle_topk_row_ordered("),
    ("ordered rows: logits row by width",
     "oracle_topk_row_ordered(logits + (int64_t)r * row_stride,",
     "oracle_topk_row_ordered(logits + (int64_t)r * width,"),
    ("ordered rows: one count slot", "ids ? ids + (int64_t)r * k : NULL, valid + r);",
     "ids ? ids + (int64_t)r * k : NULL, valid);"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, desc, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {desc}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path), str(tmp_path / "libmutant.so"))
    # In a child process: a mutant may corrupt memory (e.g. a missing clamp).
    pins = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_pins.py")
    res = subprocess.run([sys.executable, pins, lib], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, f"no pin catches the planted mistake: {desc}"
