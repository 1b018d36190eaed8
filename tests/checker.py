"""Parity of a GPU result with the oracle's, row by row.

Criteria (exact selection, order free):
* rows with n <= k: equal position by position;
* rows with n > k: the same number of -1 entries; every other entry, after
  undoing the page transform, a distinct index in [0, n); the multiset of
  selected keys (a -1 counting as the key of -inf in block mode) equal to
  the oracle's; and the index sets equal whenever the k-th key has no ties
  beyond the ones taken (count(key == T) == take).
Keys come from the oracle's own key function (pinned separately).
"""
from __future__ import annotations

import numpy as np

KEY_NEG_INF = 0x007F


def _inverse_pages(pages_row, page_size):
    inv = np.empty_like(pages_row)
    inv[pages_row] = np.arange(pages_row.size, dtype=pages_row.dtype)
    return inv


def check(orc, d, gpu_out, oracle_out, rows=None, max_report=5):
    """Return a list of failure strings (empty: parity)."""
    L, VL, k, mode = d["logits"], d["valid_len"], d["k"], d["mode"]
    width = d["width"]
    pages, P = d.get("pages"), d.get("page_size", 0)
    rows = range(L.shape[0]) if rows is None else rows
    bad = []
    for i, r in enumerate(rows):
        g = np.asarray(gpu_out[i], dtype=np.int64)
        o = np.asarray(oracle_out[i], dtype=np.int64)
        v = max(0, min(int(VL[r]), width))
        n = (v + 7) // 8 if mode == 1 else v
        if n <= k:
            if not np.array_equal(g, o):
                bad.append(f"row {r}: short row differs (n={n})")
        else:
            if pages is not None:
                npg = -(-width // P)   # entries past ceil(width / P) are never used
                inv = _inverse_pages(np.asarray(pages[r][:npg], dtype=np.int64), P)
                g = np.where(g >= 0, inv[np.maximum(g, 0) // P] * P + np.maximum(g, 0) % P, -1)
                o = np.where(o >= 0, inv[np.maximum(o, 0) // P] * P + np.maximum(o, 0) % P, -1)
            keys = orc.row_keys(L[r], v, mode).astype(np.int64)
            gs, os_ = g[g >= 0], o[o >= 0]
            if (g < 0).sum() != (o < 0).sum():
                bad.append(f"row {r}: {(g < 0).sum()} entries of -1, oracle {(o < 0).sum()}")
            elif gs.size and (gs.min() < 0 or gs.max() >= n):
                bad.append(f"row {r}: index out of range [0, {n})")
            elif np.unique(gs).size != gs.size:
                bad.append(f"row {r}: repeated indices")
            else:
                gk = np.sort(np.concatenate([keys[gs], np.full((g < 0).sum(), KEY_NEG_INF)]))
                ok = np.sort(np.concatenate([keys[os_], np.full((o < 0).sum(), KEY_NEG_INF)]))
                if not np.array_equal(gk, ok):
                    bad.append(f"row {r}: selected key multiset differs")
                else:
                    T = int(ok[0])
                    take = k - int((ok > T).sum())
                    if int((keys == T).sum()) == take and not np.array_equal(np.sort(gs),
                                                                             np.sort(os_)):
                        bad.append(f"row {r}: index set differs with no ties at T")
        if len(bad) >= max_report:
            break
    return bad
