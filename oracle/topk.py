"""Top-k selection of index rows from scores (the indexer step that produces
the index tensor).

Source: xtuner PR #2096, Main Changes item 1 -- per row, the top-k key
positions among that row's valid [start, end) range, ordered by score as
torch.topk(sorted=True) orders them, int32, and -1 for the slots a row cannot
fill (fewer valid positions than k).

Reading where the page is silent: equal scores are ordered by position,
smaller first (the page's tests avoid ties; any fixed rule makes the result
unique).
"""
from __future__ import annotations

import numpy as np


def topk_select(scores, topk: int, starts=None, ends=None) -> np.ndarray:
    """int32 [rows, topk] from float scores [rows, n]."""
    x = np.asarray(scores)
    rows, n = x.shape
    out = np.full((rows, topk), -1, dtype=np.int32)
    for r in range(rows):
        lo = 0 if starts is None else max(int(starts[r]), 0)
        hi = n if ends is None else min(int(ends[r]), n)
        if hi <= lo or topk == 0:
            continue
        pos = np.arange(lo, hi)
        order = np.lexsort((pos, -x[r, lo:hi].astype(np.float64)))   # score descending, then position
        pick = pos[order[:topk]]
        out[r, :len(pick)] = pick
    return out
