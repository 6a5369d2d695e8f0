"""Masked attention forward and backward in float64 -- the plain definitions.

Sources (by page title and section):

* MagiAttention PR #334, "BWD LoopK with warp-specialized pipeline +
  IndexSparse/BlockSparse support": Summary (the two loop orders: outer Q
  blocks / inner K blocks with dQ kept and stored once, versus outer K blocks
  with dQ accumulated), Core changes item 3 (dK/dV accumulated unscaled, then
  converted and multiplied by softmax_scale: softmax_scale sits inside the
  scores, so dQ and dK carry one factor of it and dV none).
* The backward recomputes P from Q, K and the forward LSE and produces dQ, dK,
  dV; the forward is needed only to make O and LSE.  The online-softmax
  forward recipe in the nvfp4-megamoe-kernel commit log (running max/sum,
  un-normalised P, O = acc / sum) equals the two-pass form used here in exact
  arithmetic.

Definitions (s = softmax_scale, M the mask of ``masks.py``; all sums over
pairs with M[i, j] = 1):

    S_ij  = s * q_i . k_j
    LSE_i = log sum_j exp(S_ij)                 (+inf for a row with no kept j)
    P_ij  = exp(S_ij - LSE_i)                   (0 where M = 0)
    O_i   = sum_j P_ij v_j
    D_i   = dO_i . O_i
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - D_i)
    dV_j  = sum_{h in group} sum_i P_ij dO_i
    dK_j  = s * sum_{h in group} sum_i dS_ij q_i
    dQ_i  = s * sum_j dS_ij k_j

Layouts (token-major, as the (total_q, NHK, topk) index tensor implies):
q [B,Sq,Hq,Dqk], k [B,Sk,Hk,Dqk], v [B,Sk,Hk,Dv], o/do [B,Sq,Hq,Dv],
lse [B,Hq,Sq].  Rows of a query block are handled together only because they
are independent; no sum is reordered beyond what a matrix product does.
"""
from __future__ import annotations

import numpy as np

from . import masks as _m
from .masks import MaskSpec


def _blocks(mask: MaskSpec):
    if mask.kind == "block":
        return mask.block_q, mask.block_k
    return 128, 128


def _key_positions(kbs, bk: int, seqlen_k: int) -> np.ndarray:
    if len(kbs) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(kb * bk, min((kb + 1) * bk, seqlen_k)) for kb in kbs])


def attn_fwd(q, k, v, mask: MaskSpec, causal: bool, scale: float, heads=None):
    """Forward attention in float64.  Returns (O [B,Sq,Hq,Dv], LSE [B,Hq,Sq]).

    ``heads``: optional iterable of query heads to evaluate; every other head
    is returned as an all-empty head (O = 0, LSE = +inf), which is also what an
    empty row gets.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale)
    B, Sq, Hq, _ = q.shape
    Sk, Hk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hk
    bq, bk = _blocks(mask)
    n_qb, n_kb = -(-Sq // bq), -(-Sk // bk)
    O = np.zeros((B, Sq, Hq, Dv))
    LSE = np.full((B, Hq, Sq), np.inf)
    hs = range(Hq) if heads is None else heads
    for b in range(B):
        for h in hs:
            hk = _m.kv_head(h, Hq, Hk)
            hm = _m.mask_head(h, Hq, mask) if mask.kind == "block" else 0
            for qb in range(n_qb):
                rows = np.arange(qb * bq, min((qb + 1) * bq, Sq))
                cols = _key_positions(_m.q2k_row(mask, b, hm, qb, n_qb, n_kb), bk, Sk)
                if len(cols) == 0:
                    continue
                em = _m.element_mask(rows, cols, Sq, Sk, causal) & _m.token_term(mask, b, hm, rows, cols)
                S = s * (q[b, rows, h, :] @ k[b, cols, hk, :].T)
                S = np.where(em, S, -np.inf)
                m = S.max(axis=1)
                live = np.isfinite(m)
                m_safe = np.where(live, m, 0.0)
                with np.errstate(divide="ignore"):
                    lse = m_safe + np.log(np.exp(S - m_safe[:, None]).sum(axis=1))
                lse = np.where(live, lse, np.inf)
                P = np.exp(S - lse[:, None])
                P = np.where(em & live[:, None], P, 0.0)
                O[b, rows, h, :] = P @ v[b, cols, hk, :]
                LSE[b, h, rows] = lse
    return O, LSE


def tile_grads(qr, dor, lser, dr, kc, vc, em, s):
    """P and dS for a set of query rows against a set of key columns."""
    S = s * (qr @ kc.T)
    S = np.where(em, S, -np.inf)
    with np.errstate(invalid="ignore"):
        P = np.exp(S - lser[:, None])
    P = np.where(em, P, 0.0)
    P = np.nan_to_num(P, nan=0.0)         # (-inf) - (+inf) on fully masked rows
    dP = dor @ vc.T
    dS = P * (dP - dr[:, None])
    return P, dS


def attn_bwd(q, k, v, o, do, lse, mask: MaskSpec, causal: bool, scale: float, order: str = "K",
             heads=None):
    """Backward of masked attention in float64.  Returns (dQ, dK, dV).

    ``heads``: optional iterable of query heads whose pairs are evaluated; the
    result equals the full backward when every other head's LSE is +inf
    (their P is zero, so they contribute nothing and get dQ = 0).

    order="K": for each (batch, query head, query block), for each kept key
    block of its Q->K CSR row -- accumulate dQ locally, add dK/dV per block.
    order="Q": for each (batch, KV head, key block), for each query head of the
    group and each query block of its K->Q CSR row -- accumulate dK/dV locally,
    add dQ per block.  Both orders visit exactly the same (i, j) pairs.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    s = float(scale)
    B, Sq, Hq, Dqk = q.shape
    Sk, Hk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hk
    bq, bk = _blocks(mask)
    n_qb, n_kb = -(-Sq // bq), -(-Sk // bk)
    D = np.einsum("bshd,bshd->bhs", do, o)          # D_i = dO_i . O_i   [B,Hq,Sq]
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    hset = set(range(Hq)) if heads is None else set(int(x) for x in heads)
    if order == "K":
        for b in range(B):
            for h in sorted(hset):
                hk = _m.kv_head(h, Hq, Hk)
                hm = _m.mask_head(h, Hq, mask) if mask.kind == "block" else 0
                for qb in range(n_qb):
                    rows = np.arange(qb * bq, min((qb + 1) * bq, Sq))
                    cols = _key_positions(_m.q2k_row(mask, b, hm, qb, n_qb, n_kb), bk, Sk)
                    if len(cols) == 0:
                        continue
                    em = _m.element_mask(rows, cols, Sq, Sk, causal) & _m.token_term(mask, b, hm, rows, cols)
                    qr, dor = q[b, rows, h, :], do[b, rows, h, :]
                    kc, vc = k[b, cols, hk, :], v[b, cols, hk, :]
                    P, dS = tile_grads(qr, dor, lse[b, h, rows], D[b, h, rows], kc, vc, em, s)
                    dQ[b, rows, h, :] += s * (dS @ kc)
                    dK[b, cols, hk, :] += s * (dS.T @ qr)
                    dV[b, cols, hk, :] += P.T @ dor
    elif order == "Q":
        for b in range(B):
            for hk in range(Hk):
                for kb in range(n_kb):
                    cols = np.arange(kb * bk, min((kb + 1) * bk, Sk))
                    hrow, qrow, mrow = [], [], []
                    for h in [h for h in range(Hq) if _m.kv_head(h, Hq, Hk) == hk and h in hset]:
                        hm = _m.mask_head(h, Hq, mask) if mask.kind == "block" else 0
                        for qb in _m.k2q_row(mask, b, hm, kb, n_qb, n_kb):
                            r = np.arange(qb * bq, min((qb + 1) * bq, Sq))
                            hrow.append(np.full(len(r), h))
                            mrow.append(np.full(len(r), hm))
                            qrow.append(r)
                    if not qrow:
                        continue
                    hs = np.concatenate(hrow)
                    rs = np.concatenate(qrow)
                    em = _m.element_mask(rs, cols, Sq, Sk, causal) & _m.token_term(mask, b, np.concatenate(mrow),
                                                                                   rs, cols)
                    qr, dor = q[b, rs, hs, :], do[b, rs, hs, :]
                    kc, vc = k[b, cols, hk, :], v[b, cols, hk, :]
                    P, dS = tile_grads(qr, dor, lse[b, hs, rs], D[b, hs, rs], kc, vc, em, s)
                    dK[b, cols, hk, :] += s * (dS.T @ qr)
                    dV[b, cols, hk, :] += P.T @ dor
                    np.add.at(dQ, (b, rs, hs), s * (dS @ kc))
    else:
        raise ValueError("order must be 'K' or 'Q'")
    return dQ, dK, dV


def kept_block_count(mask: MaskSpec, batch: int, heads_q: int, seqlen_q: int, seqlen_k: int,
                     causal: bool) -> int:
    """Number of (b, h, qb, kb) blocks with at least one attended pair."""
    bq, bk = _blocks(mask)
    n_qb, n_kb = -(-seqlen_q // bq), -(-seqlen_k // bk)
    n = 0
    for b in range(batch):
        for h in range(heads_q):
            hm = _m.mask_head(h, heads_q, mask) if mask.kind == "block" else 0
            for qb in range(n_qb):
                last_row = min((qb + 1) * bq, seqlen_q) - 1
                for kb in _m.q2k_row(mask, b, hm, qb, n_qb, n_kb):
                    if causal and kb * bk > last_row + seqlen_k - seqlen_q:
                        continue
                    n += 1
    return n


def flop_count(mask: MaskSpec, batch: int, heads_q: int, seqlen_q: int, seqlen_k: int,
               dim_qk: int, dim_v: int, causal: bool) -> int:
    """Backward FLOP over computed blocks: 2*(3*Dqk + 2*Dv) per pair of each kept
    block (whole blocks, diagonal blocks included; ragged edge blocks by their
    in-bounds size)."""
    bq, bk = _blocks(mask)
    n_qb, n_kb = -(-seqlen_q // bq), -(-seqlen_k // bk)
    per_pair = 2 * (3 * dim_qk + 2 * dim_v)
    total = 0
    for b in range(batch):
        for h in range(heads_q):
            hm = _m.mask_head(h, heads_q, mask) if mask.kind == "block" else 0
            for qb in range(n_qb):
                r0, r1 = qb * bq, min((qb + 1) * bq, seqlen_q)
                for kb in _m.q2k_row(mask, b, hm, qb, n_qb, n_kb):
                    if causal and kb * bk > r1 - 1 + seqlen_k - seqlen_q:
                        continue
                    c1 = min((kb + 1) * bk, seqlen_k)
                    total += (r1 - r0) * (c1 - kb * bk) * per_pair
    return total
