"""Pins for the token-exact index term of the oracle (CPU only).

Checked against things other than the oracle's own formula: torch float64
autograd over a dense mask built here by explicit loops over the index
rows, a closed form (one selected key per row: O is that key's value row and
dQ = dK = 0), the block-granular mask as the special case where every row
selects every key of its kept blocks, and finite differences.  Each test
names the mistake it catches.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(4321)


def rand(*shape):
    return RNG.standard_normal(shape)


def random_indices(B, Sq, Sk, nhk, topk, pad=0.2):
    idx = RNG.integers(0, Sk, size=(B * Sq, nhk, topk)).astype(np.int32)
    idx[RNG.random(idx.shape) < pad] = -1
    idx[RNG.random(idx.shape) < 0.05] = Sk + 3          # out of range: padding too
    return idx


def spec(idx, B, Sq, Sk, bq=4, bk=4, token=True):
    pres = oracle.indices_to_presence(idx, B, Sq, Sk, bq, bk)
    qp, qc, kp, kc = oracle.presence_to_csr(pres)
    tok = oracle.indices_to_token_mask(idx, B, Sq, Sk) if token else None
    return oracle.block_mask_from_csr(idx.shape[1], qp, qc, kp, kc, bq, bk, token=tok)


def loop_mask(idx, B, Sq, Sk, Hq, causal):
    """[B, Hq, Sq, Sk] built by plain loops over the index rows."""
    nhk = idx.shape[1]
    M = np.zeros((B, Hq, Sq, Sk), dtype=bool)
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                for j in idx[b * Sq + i, h * nhk // Hq]:
                    if 0 <= j < Sk and (not causal or j <= i + Sk - Sq):
                        M[b, h, i, j] = True
    return M


def torch_dense(q, k, v, do, M, scale):
    B, Sq, Hq, _ = q.shape
    G = Hq // k.shape[2]
    Q = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    K = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    V = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    dO = torch.tensor(do).permute(0, 2, 1, 3).contiguous()
    S = scale * Q @ K.repeat_interleave(G, dim=1).transpose(-1, -2)
    S = S.masked_fill(~torch.tensor(M), float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    P = torch.nan_to_num(torch.softmax(S, dim=-1), nan=0.0)
    O = P @ V.repeat_interleave(G, dim=1)
    (O * dO).sum().backward()
    f = lambda t: t.detach().permute(0, 2, 1, 3).numpy()
    return f(O), lse.detach().numpy(), f(Q.grad), f(K.grad), f(V.grad)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(1, 9, 11, 2, 1, 3), (2, 8, 8, 4, 2, 5), (1, 11, 7, 2, 2, 4)])
def test_token_mask_vs_torch_autograd(dims, causal):
    """Catches: the token term ignored, applied to the wrong head / transposed,
    or missing from one of the passes or loop orders."""
    B, Sq, Sk, Hq, Hk, topk = dims
    idx = random_indices(B, Sq, Sk, Hk, topk)
    mask = spec(idx, B, Sq, Sk)
    q, k, v, do = rand(B, Sq, Hq, 5), rand(B, Sk, Hk, 5), rand(B, Sk, Hk, 3), rand(B, Sq, Hq, 3)
    s = 0.52
    Ot, Lt, dqt, dkt, dvt = torch_dense(q, k, v, do, loop_mask(idx, B, Sq, Sk, Hq, causal), s)
    O, L = oracle.attn_fwd(q, k, v, mask, causal, s)
    np.testing.assert_allclose(O, Ot, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(L), np.isinf(Lt))
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], Lt[fin], atol=1e-12)
    for order in ("K", "Q"):
        dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, mask, causal, s, order=order)
        np.testing.assert_allclose(dq, dqt, atol=1e-11)
        np.testing.assert_allclose(dk, dkt, atol=1e-11)
        np.testing.assert_allclose(dv, dvt, atol=1e-11)


def test_single_selected_key_closed_form():
    """Each row selects one key j(i): P is one-hot, O_i = V_j(i),
    LSE_i = s q_i.k_j(i), dS = 0 so dQ = dK = 0, and dV_j = sum of dO_i over
    the rows that picked j.  Catches: a softmax over the whole kept block."""
    Sq, Sk, D = 6, 9, 4
    pick = np.array([3, 0, 8, 3, 5, 1])
    idx = np.full((Sq, 1, 3), -1, dtype=np.int32)
    idx[:, 0, 0] = pick
    mask = spec(idx, 1, Sq, Sk)
    q, k, v, do = rand(1, Sq, 1, D), rand(1, Sk, 1, D), rand(1, Sk, 1, D), rand(1, Sq, 1, D)
    s = 0.7
    O, L = oracle.attn_fwd(q, k, v, mask, False, s)
    np.testing.assert_allclose(O[0, :, 0], v[0, pick, 0], atol=1e-14)
    np.testing.assert_allclose(L[0, 0], s * np.einsum("id,id->i", q[0, :, 0], k[0, pick, 0]), atol=1e-13)
    dq, dk, dv = oracle.attn_bwd(q, k, v, O, do, L, mask, False, s)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    ref = np.zeros((Sk, D))
    for i, j in enumerate(pick):
        ref[j] += do[0, i, 0]
    np.testing.assert_allclose(dv[0, :, 0], ref, atol=1e-13)


def test_selecting_whole_blocks_equals_block_mask():
    """A row that selects every key of its kept blocks: token-exact and
    block-granular masks coincide.  Catches: bits cleared inside kept blocks."""
    B, Sq, Sk, bq, bk = 1, 8, 12, 4, 4
    pres = np.array([[[[1, 0, 1], [0, 1, 0]]]], dtype=np.uint8)
    rows = []
    for i in range(Sq):
        keys = [j for j in range(Sk) if pres[0, 0, i // bq, j // bk]]
        rows.append(keys + [-1] * (Sk - len(keys)))
    idx = np.asarray(rows, dtype=np.int32)[:, None, :]
    q, k, v, do = rand(B, Sq, 2, 3), rand(B, Sk, 1, 3), rand(B, Sk, 1, 2), rand(B, Sq, 2, 2)
    tok, blk = spec(idx, B, Sq, Sk, bq, bk, True), spec(idx, B, Sq, Sk, bq, bk, False)
    O1, L1 = oracle.attn_fwd(q, k, v, tok, True, 0.4)
    O2, L2 = oracle.attn_fwd(q, k, v, blk, True, 0.4)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)
    for a, b in zip(oracle.attn_bwd(q, k, v, O1, do, L1, tok, True, 0.4),
                    oracle.attn_bwd(q, k, v, O2, do, L2, blk, True, 0.4)):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_token_mask_brute_force_and_finite_differences():
    """indices_to_token_mask against the loop construction; central
    differences of sum(dO * O) under the token mask.  Catches: a wrong
    gradient on selected pairs only."""
    B, Sq, Sk, Hq, Hk = 1, 5, 6, 2, 1
    idx = random_indices(B, Sq, Sk, Hk, 3, pad=0.1)
    tok = oracle.indices_to_token_mask(idx, B, Sq, Sk)
    np.testing.assert_array_equal(tok[:, 0], loop_mask(idx, B, Sq, Sk, 1, False)[:, 0])
    mask = spec(idx, B, Sq, Sk, 2, 2)
    q, k, v, do = rand(B, Sq, Hq, 3), rand(B, Sk, Hk, 3), rand(B, Sk, Hk, 2), rand(B, Sq, Hq, 2)
    O, L = oracle.attn_fwd(q, k, v, mask, False, 0.8)
    grads = oracle.attn_bwd(q, k, v, O, do, L, mask, False, 0.8)
    eps = 1e-6
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = np.zeros_like(x)
        for idx_ in np.ndindex(*x.shape):
            ap = [q.copy(), k.copy(), v.copy()]
            am = [q.copy(), k.copy(), v.copy()]
            ap[which][idx_] += eps
            am[which][idx_] -= eps
            fp = np.sum(do * oracle.attn_fwd(*ap, mask, False, 0.8)[0])
            fm = np.sum(do * oracle.attn_fwd(*am, mask, False, 0.8)[0])
            fd[idx_] = (fp - fm) / (2 * eps)
        assert np.abs(fd - g).max() <= 1e-6 * max(np.abs(fd).max(), 1e-3)
