"""Pins for the oracle's index -> presence -> CSR converter (CPU only).

Checked against hand-derived fixtures (tests/golden/convert_small.json), a
brute force over Python sets, scipy.sparse's CSR/CSC construction (a library
routine) and invariants: transposition, permutation invariance, padding.
"""
import json
import os

import numpy as np
import pytest
import scipy.sparse as sp

import oracle


def brute_presence(indices, batch, seqlen_q, seqlen_k, bq, bk):
    """Python sets, one entry at a time."""
    nhk = indices.shape[1]
    n_qb, n_kb = -(-seqlen_q // bq), -(-seqlen_k // bk)
    sets = {}
    for r in range(indices.shape[0]):
        b, i = divmod(r, seqlen_q)
        for h in range(nhk):
            for x in indices[r, h]:
                x = int(x)
                if 0 <= x < seqlen_k:
                    sets.setdefault((b, h, i // bq), set()).add(x // bk)
    p = np.zeros((batch, nhk, n_qb, n_kb), dtype=np.uint8)
    for (b, h, qb), s in sets.items():
        for kb in s:
            p[b, h, qb, kb] = 1
    return p


def test_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "convert_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        idx = np.asarray(c["indices"], dtype=np.int32)
        p = oracle.indices_to_presence(idx, c["batch"], c["seqlen_q"], c["seqlen_k"],
                                       c["block_q"], c["block_k"])
        assert p.tolist() == c["presence"]
        qp, qc, kp, kc = oracle.presence_to_csr(p)
        assert qp.tolist() == c["q2k_row_ptr"] and qc.tolist() == c["q2k_col"]
        assert kp.tolist() == c["k2q_row_ptr"] and kc.tolist() == c["k2q_col"]


@pytest.mark.parametrize("seed", range(6))
def test_presence_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, Sq, Sk, nhk, topk = 2, int(rng.integers(1, 40)), int(rng.integers(1, 50)), 3, 5
    bq, bk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    idx = rng.integers(-3, Sk + 4, size=(B * Sq, nhk, topk)).astype(np.int32)
    p = oracle.indices_to_presence(idx, B, Sq, Sk, bq, bk)
    np.testing.assert_array_equal(p, brute_presence(idx, B, Sq, Sk, bq, bk))


@pytest.mark.parametrize("seed", range(4))
def test_csr_vs_scipy(seed):
    rng = np.random.default_rng(100 + seed)
    B, H, nq, nk = 2, 3, int(rng.integers(1, 12)), int(rng.integers(1, 12))
    p = (rng.random((B, H, nq, nk)) < 0.3).astype(np.uint8)
    qp, qc, kp, kc = oracle.presence_to_csr(p)
    ptr, col = [0], []
    tptr, tcol = [0], []
    for b in range(B):
        for h in range(H):
            m = sp.csr_matrix(p[b, h])
            m.sort_indices()
            col.extend(m.indices.tolist())
            ptr.extend((ptr[-1] + m.indptr[1:]).tolist())
            t = sp.csc_matrix(p[b, h])
            t.sort_indices()
            tcol.extend(t.indices.tolist())
            tptr.extend((tptr[-1] + t.indptr[1:]).tolist())
    assert qp.tolist() == ptr and qc.tolist() == col
    assert kp.tolist() == tptr and kc.tolist() == tcol
    assert qp.dtype == np.int32 and kc.dtype == np.int32


def test_invariants():
    rng = np.random.default_rng(5)
    B, Sq, Sk, nhk, topk = 1, 37, 53, 2, 9
    idx = rng.integers(-1, Sk, size=(B * Sq, nhk, topk)).astype(np.int32)
    p = oracle.indices_to_presence(idx, B, Sq, Sk, 8, 8)
    # permuting each row's entries changes nothing
    perm = np.take_along_axis(idx, rng.permuted(np.broadcast_to(np.arange(topk), idx.shape).copy(),
                                                axis=-1), axis=-1)
    np.testing.assert_array_equal(oracle.indices_to_presence(perm, B, Sq, Sk, 8, 8), p)
    # all -1 -> empty
    assert oracle.indices_to_presence(np.full_like(idx, -1), B, Sq, Sk, 8, 8).sum() == 0
    # out-of-range values are padding
    big = idx.copy()
    big[big < 0] = Sk + 17
    np.testing.assert_array_equal(oracle.indices_to_presence(big, B, Sq, Sk, 8, 8), p)
    # one index per row -> at most one block per row of tokens
    one = np.full_like(idx, -1)
    one[:, :, 0] = np.arange(B * Sq)[:, None] % Sk
    p1 = oracle.indices_to_presence(one, B, Sq, Sk, 1, 8)
    assert np.all(p1.sum(axis=-1) == 1)
    # the two CSRs hold the same pairs
    qp, qc, kp, kc = oracle.presence_to_csr(p)
    assert qp[-1] == kp[-1] == p.sum()
    pairs_q = set()
    n_qb, n_kb = p.shape[2], p.shape[3]
    for r in range(len(qp) - 1):
        bh, qb = divmod(r, n_qb)
        for c in qc[qp[r]:qp[r + 1]]:
            pairs_q.add((bh, qb, int(c)))
    pairs_k = set()
    for r in range(len(kp) - 1):
        bh, kb = divmod(r, n_kb)
        for c in kc[kp[r]:kp[r + 1]]:
            pairs_k.add((bh, int(c), kb))
    assert pairs_q == pairs_k


def test_full_causal_indices_give_lower_triangle():
    """Rows that select every position of [0, i] give the lower block triangle."""
    Sq = Sk = 40
    topk = Sk
    idx = np.full((Sq, 1, topk), -1, dtype=np.int32)
    for i in range(Sq):
        idx[i, 0, :i + 1] = np.arange(i + 1)
    p = oracle.indices_to_presence(idx, 1, Sq, Sk, 8, 8)
    np.testing.assert_array_equal(p[0, 0], np.tril(np.ones((5, 5), dtype=np.uint8)))
