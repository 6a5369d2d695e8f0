"""Pins for the top-k selection oracle (CPU only): torch.topk(sorted=True) on
unique scores (a library routine), brute force by sorting each row's valid
range, and the special cases the page names (rows with fewer valid values
than k, packed causal ranges).  Catches: an off-by-one range end, ascending
order, a missing -1 pad, positions relative to the range start."""
import numpy as np
import torch

import oracle

RNG = np.random.default_rng(77)


def unique_scores(rows, n):
    x = RNG.permutation(rows * n).reshape(rows, n).astype(np.float32) / (rows * n) - 0.5
    return x


def test_matches_torch_topk_on_unique_scores():
    x = unique_scores(6, 50)
    got = oracle.topk_select(x, 9)
    ref = torch.topk(torch.from_numpy(x), 9, dim=1, sorted=True).indices.numpy()
    np.testing.assert_array_equal(got, ref)


def test_ranges_fewer_than_k_and_empty_rows():
    x = unique_scores(5, 20)
    starts = np.array([0, 5, 10, 7, 3])
    ends = np.array([20, 9, 10, 30, 2])
    got = oracle.topk_select(x, 6, starts, ends)
    for r in range(5):
        lo, hi = starts[r], min(ends[r], 20)
        pos = [p for p in range(lo, hi)]
        best = sorted(pos, key=lambda p: -x[r, p])[:6]
        assert list(got[r, :len(best)]) == best
        assert np.all(got[r, len(best):] == -1)
    assert np.all(got[2] == -1) and np.all(got[4] == -1)


def test_packed_causal_ranges():
    """Two packed sequences of 5 and 7 tokens: row i of a sequence starting at
    s sees [s, i + 1)."""
    lens = [5, 7]
    starts, ends = [], []
    s = 0
    for L in lens:
        for i in range(L):
            starts.append(s)
            ends.append(s + i + 1)
        s += L
    x = unique_scores(12, 12)
    got = oracle.topk_select(x, 3, np.array(starts), np.array(ends))
    for r in range(12):
        cand = np.arange(starts[r], ends[r])
        ref = cand[np.argsort(-x[r, cand], kind="stable")][:3]
        assert list(got[r, :len(ref)]) == list(ref)
        assert np.all(got[r, len(ref):] == -1)


def test_ties_resolve_to_smaller_position():
    x = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.topk_select(x, 4), [[1, 2, 4, 3]])
