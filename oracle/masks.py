"""Which (query, key) pairs an attention head attends.

M[b, h, i, j] is the AND of three terms:

1. the mask kind -- dense: always 1; block CSR: 1 iff key block j // block_k is
   listed in the Q->K CSR row of (b, mask head, query block i // block_q).
   This is the "per M-block, list of N-blocks" form of MagiAttention PR #334
   (Core changes, item 2, prepare_block_sparse_bwd_loopk).
2. if causal: j <= i + Sk - Sq (bottom-right alignment; with Sq == Sk it is the
   usual lower triangle).  The pages name causal runs without fixing the
   alignment; bottom-right is the reading taken here.
3. bounds: i < Sq and j < Sk.  A last block shorter than block_q/block_k covers
   the remainder of the sequence.

Readings where the pages are silent:

* mask heads ``Hm`` may be 1, Hk or Hq; query head h uses mask head
  ``h * Hm // Hq`` (so with Hm == Hk the query heads of one GQA group share the
  KV head's mask, which is how token indices of shape (total_q, NHK, topk)
  -- PR #334, Core changes item 2 -- are laid out).
* GQA: query head h reads KV head ``h // (Hq // Hk)`` (consecutive query
  heads share a KV head).
* inside a kept block every pair is attended (the index path is block-granular:
  PR #334 routes index sparsity through the block-sparse machinery) -- unless
  the mask carries a token mask: then a fourth term ANDs in token[b, hm, i, j],
  query i attending exactly the keys its index row selected (the token-exact
  reading of DSA sparsity, xtuner PR #2096 Background: each query keeps its
  top-k key positions).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class MaskSpec:
    kind: str                                   # "dense" or "block"
    heads: int = 0                              # Hm (block masks only)
    block_q: int = 128
    block_k: int = 128
    q2k_row_ptr: Optional[np.ndarray] = None    # int [B*Hm*nQB + 1]
    q2k_col: Optional[np.ndarray] = None        # int [nnz], ascending per row
    k2q_row_ptr: Optional[np.ndarray] = None    # int [B*Hm*nKB + 1]
    k2q_col: Optional[np.ndarray] = None        # int [nnz], ascending per row
    token: Optional[np.ndarray] = None          # bool [B, Hm, Sq, Sk]: token-exact term, or None


def dense_mask() -> MaskSpec:
    return MaskSpec(kind="dense")


def block_mask_from_csr(heads: int, q2k_row_ptr, q2k_col, k2q_row_ptr=None, k2q_col=None,
                        block_q: int = 128, block_k: int = 128, token=None) -> MaskSpec:
    return MaskSpec(kind="block", heads=heads, block_q=block_q, block_k=block_k,
                    token=None if token is None else np.asarray(token, dtype=bool),
                    q2k_row_ptr=np.asarray(q2k_row_ptr, dtype=np.int64),
                    q2k_col=np.asarray(q2k_col, dtype=np.int64),
                    k2q_row_ptr=None if k2q_row_ptr is None else np.asarray(k2q_row_ptr, dtype=np.int64),
                    k2q_col=None if k2q_col is None else np.asarray(k2q_col, dtype=np.int64))


def kv_head(h: int, heads_q: int, heads_k: int) -> int:
    """KV head read by query head h (consecutive query heads share a KV head)."""
    return h // (heads_q // heads_k)


def mask_head(h: int, heads_q: int, mask: MaskSpec) -> int:
    """Mask head used by query head h."""
    return h * mask.heads // heads_q


def q2k_row(mask: MaskSpec, b: int, hm: int, qb: int, n_qb: int, n_kb: int) -> np.ndarray:
    """Key blocks kept for query block qb of (batch b, mask head hm), ascending."""
    if mask.kind == "dense":
        return np.arange(n_kb)
    r = (b * mask.heads + hm) * n_qb + qb
    return mask.q2k_col[mask.q2k_row_ptr[r]:mask.q2k_row_ptr[r + 1]]


def k2q_row(mask: MaskSpec, b: int, hm: int, kb: int, n_qb: int, n_kb: int) -> np.ndarray:
    """Query blocks kept for key block kb of (batch b, mask head hm), ascending."""
    if mask.kind == "dense":
        return np.arange(n_qb)
    r = (b * mask.heads + hm) * n_kb + kb
    return mask.k2q_col[mask.k2q_row_ptr[r]:mask.k2q_row_ptr[r + 1]]


def element_mask(rows: np.ndarray, cols: np.ndarray, seqlen_q: int, seqlen_k: int,
                 causal: bool) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: the causal and bounds terms for the given
    query positions ``rows`` and key positions ``cols`` (block membership is
    decided by the caller, which only passes keys of kept blocks)."""
    r = np.asarray(rows)[:, None]
    c = np.asarray(cols)[None, :]
    m = (r < seqlen_q) & (c < seqlen_k)
    if causal:
        m &= c <= r + (seqlen_k - seqlen_q)
    return m


def token_term(mask: MaskSpec, b: int, hm, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """The token-exact term for query positions ``rows`` (with mask heads
    ``hm``, a scalar or one per row) and key positions ``cols``: all True
    when the mask has no token mask."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    if mask.token is None:
        return np.ones((len(rows), len(cols)), dtype=bool)
    hm = np.broadcast_to(np.asarray(hm), rows.shape)
    return mask.token[b, hm[:, None], rows[:, None], cols[None, :]]


def full_mask(mask: MaskSpec, b: int, h: int, heads_q: int, seqlen_q: int, seqlen_k: int,
              causal: bool) -> np.ndarray:
    """Boolean [Sq, Sk] mask of (b, h): all three terms.  For tiny shapes and tests."""
    bq = mask.block_q if mask.kind == "block" else 128
    bk = mask.block_k if mask.kind == "block" else 128
    n_qb = -(-seqlen_q // bq)
    n_kb = -(-seqlen_k // bk)
    kind = np.zeros((seqlen_q, seqlen_k), dtype=bool)
    hm = mask_head(h, heads_q, mask) if mask.kind == "block" else 0
    for qb in range(n_qb):
        for kb in q2k_row(mask, b, hm, qb, n_qb, n_kb):
            kind[qb * bq:(qb + 1) * bq, kb * bk:(kb + 1) * bk] = True
    r, c = np.arange(seqlen_q), np.arange(seqlen_k)
    return kind & element_mask(r, c, seqlen_q, seqlen_k, causal) & token_term(mask, b, hm, r, c)
