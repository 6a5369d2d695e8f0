"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself: hand-derived worked
examples (tests/golden), closed forms, finite differences of its own forward,
torch autograd in float64 over an independently built dense mask (a library
routine), and structural identities (GQA == repeated-KV MHA, dense == all-kept
CSR, the two loop orders, sum rules).  Each test names the mistake it is meant
to catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.masks import MaskSpec, full_mask

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def block_spec(presence, bq, bk):
    qp, qc, kp, kc = oracle.presence_to_csr(presence)
    return oracle.block_mask_from_csr(presence.shape[1], qp, qc, kp, kc, bq, bk)


def torch_reference(q, k, v, do, presence, bq, bk, causal, scale):
    """Dense masked attention in float64 with torch autograd.

    The mask is built here from library routines (np.kron for blocks,
    torch.tril with a diagonal offset for bottom-right causal,
    repeat_interleave for GQA), independently of oracle/masks.py."""
    B, Sq, Hq, _ = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    G = Hq // Hk
    Q = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    K = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    V = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    dO = torch.tensor(do).permute(0, 2, 1, 3).contiguous()
    M = torch.ones(B, Hq, Sq, Sk, dtype=torch.bool)
    if presence is not None:
        Hm = presence.shape[1]
        for b in range(B):
            for h in range(Hq):
                hm = h // (Hq // Hm)
                blk = np.kron(presence[b, hm], np.ones((bq, bk), dtype=np.uint8))[:Sq, :Sk]
                M[b, h] &= torch.tensor(blk.astype(bool))
    if causal:
        M &= torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
    Kr = K.repeat_interleave(G, dim=1)
    Vr = V.repeat_interleave(G, dim=1)
    S = scale * Q @ Kr.transpose(-1, -2)
    S = S.masked_fill(~M, float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    P = torch.softmax(S, dim=-1)
    P = torch.nan_to_num(P, nan=0.0)
    O = P @ Vr
    (O * dO).sum().backward()
    bshd = lambda t: t.detach().permute(0, 2, 1, 3).numpy()
    return bshd(O), lse.detach().numpy(), bshd(Q.grad), bshd(K.grad), bshd(V.grad)


def load_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)
    arr = lambda key: np.asarray(g[key], dtype=np.float64)
    return g, arr


# ----------------------------------------------------------------------------
# hand-derived worked examples
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["attn_two_keys.json", "attn_causal_bottom_right.json",
                                  "attn_gqa_head_map.json", "attn_block_sparse.json"])
@pytest.mark.parametrize("order", ["K", "Q"])
def test_golden_worked_examples(golden_dir, name, order):
    """Catches: misplaced softmax_scale, wrong sign in dS, top-left causal,
    interleaved GQA map, transposed block presence."""
    g, arr = load_golden(golden_dir, name)
    q, k, v, do = arr("q"), arr("k"), arr("v"), arr("do")
    if "presence" in g:
        blk = g["block"]
        mask = oracle.block_mask_from_csr(g["mask_heads"], g["q2k_row_ptr"], g["q2k_col"],
                                          g["k2q_row_ptr"], g["k2q_col"], blk, blk)
    else:
        mask = oracle.dense_mask()
    O, L = oracle.attn_fwd(q, k, v, mask, g["causal"], g["scale"])
    e = g["expected"]
    np.testing.assert_allclose(O, np.asarray(e["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.asarray(e["lse"]), rtol=0, atol=1e-12)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, mask, g["causal"], g["scale"], order=order)
    np.testing.assert_allclose(dq, np.asarray(e["dq"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, np.asarray(e["dk"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, np.asarray(e["dv"]), rtol=0, atol=1e-12)


def test_golden_block_csr_matches_presence(golden_dir):
    g, _ = load_golden(golden_dir, "attn_block_sparse.json")
    qp, qc, kp, kc = oracle.presence_to_csr(np.asarray(g["presence"]))
    assert qp.tolist() == g["q2k_row_ptr"] and qc.tolist() == g["q2k_col"]
    assert kp.tolist() == g["k2q_row_ptr"] and kc.tolist() == g["k2q_col"]


# ----------------------------------------------------------------------------
# forward: closed forms and library cross-check
# ----------------------------------------------------------------------------
def test_forward_zero_query_is_uniform():
    """Q = 0: P uniform over visible keys, LSE_i = ln n_i, O_i = mean of visible v_j.
    Catches: log base, causal alignment, missing normalisation."""
    B, Sq, Sk, H, D = 1, 6, 9, 2, 3
    q = np.zeros((B, Sq, H, D))
    k, v = rand(B, Sk, H, D), rand(B, Sk, H, 5)
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), True, 0.7)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        np.testing.assert_allclose(L[0, :, i], math.log(n), atol=1e-13)
        np.testing.assert_allclose(O[0, i], v[0, :n].mean(axis=0), atol=1e-13)


def test_forward_single_key():
    """Sk = 1: LSE = s*q.k and O = v.  Catches: scale applied outside the exponent."""
    q, k, v = rand(2, 4, 3, 8), rand(2, 1, 3, 8), rand(2, 1, 3, 2)
    s = 0.37
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), False, s)
    np.testing.assert_allclose(L, s * np.einsum("bshd,bhd->bhs", q, k[:, 0]), atol=1e-13)
    np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), atol=1e-13)


def test_forward_rows_normalised():
    """sum_j P_ij = 1: with v = 1 every non-empty row of O is exactly 1."""
    q, k = rand(1, 11, 4, 6), rand(1, 13, 2, 6)
    v = np.ones((1, 13, 2, 1))
    pres = (RNG.random((1, 4, 3, 4)) < 0.5).astype(np.uint8)
    pres[:, :, 0, 0] = 1
    O, L = oracle.attn_fwd(q, k, v, block_spec(pres, 4, 4), False, 0.5)
    live = np.isfinite(L).transpose(0, 2, 1)
    np.testing.assert_allclose(O[..., 0][live], 1.0, atol=1e-13)
    assert np.all(O[..., 0][~live] == 0.0)


@pytest.mark.parametrize("case", [
    dict(B=2, Sq=7, Sk=7, Hq=2, Hk=2, causal=False, block=None),
    dict(B=1, Sq=5, Sk=9, Hq=4, Hk=2, causal=True, block=None),
    dict(B=1, Sq=9, Sk=5, Hq=2, Hk=1, causal=True, block=None),
    dict(B=2, Sq=10, Sk=7, Hq=4, Hk=2, causal=False, block=(3, 2, "Hq")),
    dict(B=1, Sq=8, Sk=11, Hq=6, Hk=2, causal=True, block=(4, 3, "Hk")),
    dict(B=1, Sq=6, Sk=6, Hq=2, Hk=2, causal=False, block=(2, 2, "1")),
])
def test_forward_backward_vs_torch_autograd(case):
    """Library cross-check of O, LSE, dQ, dK, dV (torch float64 autograd over a
    dense masked softmax).  Catches: any arithmetic slip in either pass."""
    B, Sq, Sk, Hq, Hk = case["B"], case["Sq"], case["Sk"], case["Hq"], case["Hk"]
    Dqk, Dv, s = 5, 3, 0.45
    q, k, v, do = rand(B, Sq, Hq, Dqk), rand(B, Sk, Hk, Dqk), rand(B, Sk, Hk, Dv), rand(B, Sq, Hq, Dv)
    presence, bq, bk = None, 128, 128
    if case["block"] is None:
        mask = oracle.dense_mask()
    else:
        bq, bk, hsel = case["block"]
        Hm = {"Hq": Hq, "Hk": Hk, "1": 1}[hsel]
        presence = (RNG.random((B, Hm, -(-Sq // bq), -(-Sk // bk))) < 0.5).astype(np.uint8)
        mask = block_spec(presence, bq, bk)
    O, L = oracle.attn_fwd(q, k, v, mask, case["causal"], s)
    Ot, Lt, dqt, dkt, dvt = torch_reference(q, k, v, do, presence, bq, bk, case["causal"], s)
    np.testing.assert_allclose(O, Ot, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(L), np.isinf(Lt))
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], Lt[fin], atol=1e-12)
    for order in ("K", "Q"):
        dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, mask, case["causal"], s, order=order)
        np.testing.assert_allclose(dq, dqt, atol=1e-11)
        np.testing.assert_allclose(dk, dkt, atol=1e-11)
        np.testing.assert_allclose(dv, dvt, atol=1e-11)


# ----------------------------------------------------------------------------
# backward: finite differences of the oracle's own forward
# ----------------------------------------------------------------------------
def _fd_check(q, k, v, do, mask, causal, s):
    def loss(q_, k_, v_):
        O, _ = oracle.attn_fwd(q_, k_, v_, mask, causal, s)
        return float(np.sum(do * O))

    O, L = oracle.attn_fwd(q, k, v, mask, causal, s)
    grads = oracle.attn_bwd(q, k, v, O, do, L, mask, causal, s, order="K")
    eps = 1e-6
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        scale = max(np.abs(fd).max(), 1e-3)
        assert np.abs(fd - g).max() <= 1e-6 * scale, (which, np.abs(fd - g).max(), scale)


@pytest.mark.parametrize("kind", ["dense", "dense_causal", "block_Hq", "block_Hk", "block_1",
                                  "block_causal", "causal_sq_gt_sk"])
def test_backward_finite_differences(kind):
    """Central differences of L = sum(dO * O(Q, K, V)) with the mask fixed.
    Catches: a dropped term, wrong sign, wrong index or a transposed operand in
    any of dQ, dK, dV."""
    B, Hq, Hk, Sq, Sk, Dqk, Dv = 1, 2, 1, 5, 7, 4, 3
    causal = kind in ("dense_causal", "block_causal", "causal_sq_gt_sk")
    if kind == "causal_sq_gt_sk":
        Sq, Sk = 7, 5
    q, k, v, do = rand(B, Sq, Hq, Dqk), rand(B, Sk, Hk, Dqk), rand(B, Sk, Hk, Dv), rand(B, Sq, Hq, Dv)
    if kind.startswith("block"):
        Hm = {"block_Hq": Hq, "block_Hk": Hk, "block_1": 1, "block_causal": Hq}[kind]
        pres = (RNG.random((B, Hm, 3, 4)) < 0.6).astype(np.uint8)
        pres[:, :, :, 0] = 1
        mask = block_spec(pres, 2, 2)
    else:
        mask = oracle.dense_mask()
    _fd_check(q, k, v, do, mask, causal, 0.61)


# ----------------------------------------------------------------------------
# backward: closed forms, sum rules, structural identities
# ----------------------------------------------------------------------------
def test_sum_rules():
    """rowsum(dS) = 0 per query (with unrounded O and LSE) implies
    sum_j dK_j = 0 and sum_j dV_j = sum over non-empty rows of dO, per (b, KV head)."""
    B, Hq, Hk, Sq, Sk = 2, 4, 2, 9, 12
    q, k, v, do = rand(B, Sq, Hq, 6), rand(B, Sk, Hk, 6), rand(B, Sk, Hk, 4), rand(B, Sq, Hq, 4)
    pres = (RNG.random((B, Hq, 3, 4)) < 0.5).astype(np.uint8)
    mask = block_spec(pres, 4, 3)
    O, L = oracle.attn_fwd(q, k, v, mask, False, 0.4)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, mask, False, 0.4)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    live = np.isfinite(L).transpose(0, 2, 1)[..., None]        # [B,Sq,Hq,1]
    dsum = np.where(live, do, 0.0).reshape(B, Sq, Hk, Hq // Hk, 4).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), dsum, atol=1e-12)


def test_identical_value_rows_give_zero_dq_dk():
    """All v_j equal -> dP_ij = D_i -> dS = 0 -> dQ = dK = 0 (dV stays nonzero)."""
    q, k, do = rand(1, 6, 2, 4), rand(1, 8, 2, 4), rand(1, 6, 2, 3)
    v = np.broadcast_to(rand(1, 1, 2, 3), (1, 8, 2, 3)).copy()
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), True, 0.5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, oracle.dense_mask(), True, 0.5)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    assert np.abs(dv).max() > 0.1


def test_single_key_backward():
    """Sk = 1: dQ = dK = 0 and dV = sum_i dO_i."""
    q, k, v, do = rand(1, 5, 3, 4), rand(1, 1, 3, 4), rand(1, 1, 3, 2), rand(1, 5, 3, 2)
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), False, 0.5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, oracle.dense_mask(), False, 0.5)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv[:, 0], do.sum(axis=1), atol=1e-13)


def test_zero_query_dq_closed_form():
    """Q = 0, dense non-causal: P = 1/Sk, dQ_i = s/Sk * sum_j (dO_i.(v_j - O_i)) k_j."""
    Sq, Sk, s = 4, 6, 0.8
    q = np.zeros((1, Sq, 1, 3))
    k, v, do = rand(1, Sk, 1, 3), rand(1, Sk, 1, 2), rand(1, Sq, 1, 2)
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), False, s)
    dq, _, _ = oracle.attn_bwd(q, k, v, O, do, L, oracle.dense_mask(), False, s)
    vbar = v[0, :, 0].mean(axis=0)
    for i in range(Sq):
        w = (v[0, :, 0] - vbar) @ do[0, i, 0]              # dP_ij - D_i
        np.testing.assert_allclose(dq[0, i, 0], s / Sk * (w @ k[0, :, 0]), atol=1e-13)


def test_gqa_equals_repeated_mha():
    """GQA result == MHA with K/V repeated per group (consecutive heads) and
    dK/dV summed over the group."""
    B, Hq, Hk, Sq, Sk = 1, 6, 2, 7, 10
    G = Hq // Hk
    q, k, v, do = rand(B, Sq, Hq, 4), rand(B, Sk, Hk, 4), rand(B, Sk, Hk, 3), rand(B, Sq, Hq, 3)
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    m = oracle.dense_mask()
    O1, L1 = oracle.attn_fwd(q, k, v, m, True, 0.5)
    O2, L2 = oracle.attn_fwd(q, kr, vr, m, True, 0.5)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    g1 = oracle.attn_bwd(q, k, v, O1, do, L1, m, True, 0.5)
    g2 = oracle.attn_bwd(q, kr, vr, O2, do, L2, m, True, 0.5)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(B, Sk, Hk, G, 4).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(g1[2], g2[2].reshape(B, Sk, Hk, G, 3).sum(axis=3), atol=1e-13)


def test_mask_head_map():
    """A mask with Hm = Hk equals the Hm = Hq mask that repeats each KV head's
    presence over its query group (query head h uses mask head h*Hm//Hq)."""
    B, Hq, Hk, Sq, Sk = 1, 4, 2, 8, 8
    q, k, v, do = rand(B, Sq, Hq, 4), rand(B, Sk, Hk, 4), rand(B, Sk, Hk, 3), rand(B, Sq, Hq, 3)
    pres = (RNG.random((B, Hk, 4, 4)) < 0.5).astype(np.uint8)
    pres[:, 0] = 1 - pres[:, 1]          # the two KV heads' masks differ in every block
    pres[..., 0] = 1
    m1 = block_spec(pres, 2, 2)
    m2 = block_spec(np.repeat(pres, Hq // Hk, axis=1), 2, 2)
    O1, L1 = oracle.attn_fwd(q, k, v, m1, False, 0.5)
    O2, L2 = oracle.attn_fwd(q, k, v, m2, False, 0.5)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    for a, b in zip(oracle.attn_bwd(q, k, v, O1, do, L1, m1, False, 0.5, "Q"),
                    oracle.attn_bwd(q, k, v, O2, do, L2, m2, False, 0.5, "Q")):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_dense_equals_all_kept_csr_and_lower_triangle_equals_causal():
    B, Hq, Hk, S = 1, 2, 2, 12
    q, k, v, do = rand(B, S, Hq, 4), rand(B, S, Hk, 4), rand(B, S, Hk, 3), rand(B, S, Hq, 3)
    full = np.ones((B, Hq, 4, 4), dtype=np.uint8)
    lower = np.tril(full)
    d = oracle.dense_mask()
    for (m_a, c_a), (m_b, c_b) in [((d, False), (block_spec(full, 3, 3), False)),
                                   ((d, True), (block_spec(lower, 3, 3), True))]:
        Oa, La = oracle.attn_fwd(q, k, v, m_a, c_a, 0.5)
        Ob, Lb = oracle.attn_fwd(q, k, v, m_b, c_b, 0.5)
        np.testing.assert_allclose(Oa, Ob, atol=1e-13)
        np.testing.assert_allclose(La, Lb, atol=1e-13)
        for x, y in zip(oracle.attn_bwd(q, k, v, Oa, do, La, m_a, c_a, 0.5),
                        oracle.attn_bwd(q, k, v, Ob, do, Lb, m_b, c_b, 0.5, "Q")):
            np.testing.assert_allclose(x, y, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_k_order_equals_q_order(seed):
    """Both loop orders visit the same pairs: results agree to rounding."""
    rng = np.random.default_rng(seed)
    B, Hq, Hk, Sq, Sk = 2, 4, 2, 13, 10
    q, k, v, do = (rng.standard_normal(s) for s in [(B, Sq, Hq, 5), (B, Sk, Hk, 5),
                                                     (B, Sk, Hk, 3), (B, Sq, Hq, 3)])
    Hm = [1, Hk, Hq][seed]
    pres = (rng.random((B, Hm, 4, 3)) < 0.5).astype(np.uint8)
    mask = block_spec(pres, 4, 4)
    causal = seed == 2
    O, L = oracle.attn_fwd(q, k, v, mask, causal, 0.3)
    gk = oracle.attn_bwd(q, k, v, O, do, L, mask, causal, 0.3, "K")
    gq = oracle.attn_bwd(q, k, v, O, do, L, mask, causal, 0.3, "Q")
    for a, b in zip(gk, gq):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_empty_rows():
    """Sq > Sk causal: rows with no visible key get LSE = +inf, O = 0, dQ = 0."""
    q, k, v, do = rand(1, 6, 1, 3), rand(1, 3, 1, 3), rand(1, 3, 1, 2), rand(1, 6, 1, 2)
    O, L = oracle.attn_fwd(q, k, v, oracle.dense_mask(), True, 0.5)
    assert np.all(np.isinf(L[0, 0, :3])) and np.all(np.isfinite(L[0, 0, 3:]))
    assert np.all(O[0, :3] == 0)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, oracle.dense_mask(), True, 0.5)
    assert np.all(dq[0, :3] == 0)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))


def test_heads_subset_forward():
    """attn_fwd(heads=...) evaluates the listed heads exactly and leaves the
    others empty (O = 0, LSE = +inf)."""
    q, k, v = rand(1, 5, 4, 3), rand(1, 5, 2, 3), rand(1, 5, 2, 2)
    Oa, La = oracle.attn_fwd(q, k, v, oracle.dense_mask(), True, 0.5)
    Ob, Lb = oracle.attn_fwd(q, k, v, oracle.dense_mask(), True, 0.5, heads=[1, 2])
    np.testing.assert_array_equal(Ob[:, :, [1, 2]], Oa[:, :, [1, 2]])
    np.testing.assert_array_equal(Lb[:, [1, 2]], La[:, [1, 2]])
    assert np.all(Ob[:, :, [0, 3]] == 0) and np.all(np.isinf(Lb[:, [0, 3]]))


def test_full_mask_against_kron():
    """oracle.masks.full_mask agrees with a Kronecker expansion + tril."""
    pres = (RNG.random((1, 2, 3, 4)) < 0.5).astype(np.uint8)
    mask = block_spec(pres, 3, 2)
    for causal in (False, True):
        for h in range(4):
            m = full_mask(mask, 0, h, 4, 8, 7, causal)
            ref = np.kron(pres[0, h // 2], np.ones((3, 2), dtype=np.uint8))[:8, :7].astype(bool)
            if causal:
                ref &= np.tril(np.ones((8, 7), dtype=bool), k=7 - 8)
            np.testing.assert_array_equal(m, ref)


def test_flop_and_block_counts():
    """Counting convention: whole computed blocks, 2*(3*Dqk + 2*Dv) per pair."""
    d = oracle.dense_mask()
    # causal 4x4 blocks of 128: 10 computed blocks per head
    assert oracle.kept_block_count(d, 1, 2, 512, 512, True) == 20
    assert oracle.flop_count(d, 1, 2, 512, 512, 128, 128, True) == 20 * 128 * 128 * 2 * 640
    # ragged: Sq=Sk=200 dense non-causal -> pairs = 200*200
    assert oracle.flop_count(d, 1, 1, 200, 200, 64, 64, False) == 200 * 200 * 2 * 320
    # block mask: count = nnz * (Hq / Hm)
    pres = np.array([[[[1, 0], [1, 1]]]], dtype=np.uint8)
    m = block_spec(pres, 128, 128)
    assert oracle.kept_block_count(m, 1, 4, 256, 256, False) == 12
    # 192/128 dims
    assert oracle.flop_count(d, 1, 1, 128, 128, 192, 128, True) == 128 * 128 * 2 * (3 * 192 + 2 * 128)


def test_heads_subset_backward_matches_infinite_lse():
    """attn_bwd(heads=...) equals the full backward when every other head has
    LSE = +inf (such heads contribute nothing and get dQ = 0)."""
    B, Hq, Hk, Sq, Sk = 1, 4, 2, 9, 11
    q, k, v, do = rand(B, Sq, Hq, 4), rand(B, Sk, Hk, 4), rand(B, Sk, Hk, 3), rand(B, Sq, Hq, 3)
    m = oracle.dense_mask()
    O, L = oracle.attn_fwd(q, k, v, m, True, 0.5, heads=[1, 2])
    full = oracle.attn_bwd(q, k, v, O, do, L, m, True, 0.5)
    sub = oracle.attn_bwd(q, k, v, O, do, L, m, True, 0.5, heads=[1, 2])
    subq = oracle.attn_bwd(q, k, v, O, do, L, m, True, 0.5, order="Q", heads=[1, 2])
    for a, b, c in zip(full, sub, subq):
        np.testing.assert_allclose(a, b, atol=1e-13)
        np.testing.assert_allclose(a, c, atol=1e-12)
    assert np.all(full[0][:, :, [0, 3]] == 0)
