"""GPU top-k selection against the oracle: exact equality (positions are
unique once ties resolve to the smaller position), over normal and
concentrated score distributions, packed causal ranges, rows with fewer valid
positions than k, ties and large k."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def run(x, k, starts=None, ends=None):
    import index_sparse_attention_amd as isa
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda() if a is not None else None
    got = isa.topk_select(t(x), k, t(starts), t(ends))
    torch.cuda.synchronize()
    return got.cpu().numpy()


def packed_causal(lens):
    starts, ends, s = [], [], 0
    for L in lens:
        for i in range(L):
            starts.append(s)
            ends.append(s + i + 1)
        s += L
    return np.array(starts, dtype=np.int32), np.array(ends, dtype=np.int32)


@pytest.mark.parametrize("dist", ["normal", "concentrated", "ties"])
@pytest.mark.parametrize("k", [1, 64, 300, 2048])
def test_topk_full_rows(dist, k):
    g = synth.seed_streams(90 + k)[0]
    rows, n = 37, 3000
    x = g.standard_normal((rows, n)).astype(np.float32)
    if dist == "concentrated":
        x = (1.0 + 1e-6 * x).astype(np.float32)            # nearly all keys share their top bits
    if dist == "ties":
        x = np.round(x * 4).astype(np.float32)             # many equal scores
    log(f"topk full rows dist={dist} k={k}")
    np.testing.assert_array_equal(run(x, k), oracle.topk_select(x, k))


@pytest.mark.parametrize("k", [16, 512])
def test_topk_packed_causal_ranges(k):
    g = synth.seed_streams(95)[0]
    lens = [700, 1, 1500, 300]
    starts, ends = packed_causal(lens)
    n = sum(lens)
    x = g.standard_normal((n, n)).astype(np.float32)
    log(f"topk packed causal k={k}")
    np.testing.assert_array_equal(run(x, k, starts, ends), oracle.topk_select(x, k, starts, ends))


def test_topk_ranges_edge_cases():
    g = synth.seed_streams(96)[0]
    x = g.standard_normal((6, 1000)).astype(np.float32)
    starts = np.array([0, 10, 500, 999, -5, 700], dtype=np.int32)
    ends = np.array([1000, 10, 400, 1200, 3, 720], dtype=np.int32)
    np.testing.assert_array_equal(run(x, 64, starts, ends), oracle.topk_select(x, 64, starts, ends))
