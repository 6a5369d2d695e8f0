"""Token top-k indices -> block presence -> Q->K and K->Q CSR lists.

Sources:

* MagiAttention PR #334, Core changes item 2: token-level indices of shape
  (total_q, NHK, topk) become block-level sparsity by scattering into a
  presence matrix; the forward-direction normalisation then lists, for each
  query block (M-block), its key blocks (N-blocks).
* MagiAttention PR #331, Summary and "CSR Tile Mapping": the backward also
  uses K->Q ("K2Q") CSR metadata, i.e. for each key block the list of query
  blocks -- the transpose of the Q->K lists.
* xtuner PR #2096, Main Changes item 1: the index producer returns int32
  indices and marks invalid positions with -1.

Readings where the pages are silent:

* total_q = B * Sq; row r is query i = r mod Sq of sequence b = r // Sq, and
  an index value is a key position inside sequence b (non-varlen).
* -1, and any other value outside [0, Sk), is padding and selects nothing;
  duplicates select once; the order of a row's entries does not matter.
* presence[b, hk, qb, kb] = 1 iff some row of query block qb (rows
  qb*block_q .. min((qb+1)*block_q, Sq)-1) has an index in key block kb.
* CSR rows are flattened over (b, head) then block, columns ascending,
  row_ptr[0] = 0, int32.
"""
from __future__ import annotations

import numpy as np


def indices_to_presence(indices, batch: int, seqlen_q: int, seqlen_k: int,
                        block_q: int = 128, block_k: int = 128) -> np.ndarray:
    """uint8 presence [B, NHK, nQB, nKB] from int indices [B*Sq, NHK, topk]."""
    idx = np.asarray(indices)
    assert idx.ndim == 3 and idx.shape[0] == batch * seqlen_q
    nhk = idx.shape[1]
    n_qb, n_kb = -(-seqlen_q // block_q), -(-seqlen_k // block_k)
    pres = np.zeros((batch, nhk, n_qb, n_kb), dtype=np.uint8)
    for b in range(batch):
        rows = idx[b * seqlen_q:(b + 1) * seqlen_q].astype(np.int64)    # [Sq, NHK, topk]
        qb = (np.arange(seqlen_q) // block_q)[:, None, None]
        hk = np.arange(nhk)[None, :, None]
        valid = (rows >= 0) & (rows < seqlen_k)
        qb_b = np.broadcast_to(qb, rows.shape)[valid]
        hk_b = np.broadcast_to(hk, rows.shape)[valid]
        kb_b = rows[valid] // block_k
        pres[b, hk_b, qb_b, kb_b] = 1
    return pres


def indices_to_token_mask(indices, batch: int, seqlen_q: int, seqlen_k: int) -> np.ndarray:
    """bool [B, NHK, Sq, Sk]: query i of sequence b attends key j for KV head
    hk iff j appears in its index row (the token-exact reading; same padding
    rules as indices_to_presence)."""
    idx = np.asarray(indices)
    assert idx.ndim == 3 and idx.shape[0] == batch * seqlen_q
    nhk = idx.shape[1]
    tok = np.zeros((batch, nhk, seqlen_q, seqlen_k), dtype=bool)
    for b in range(batch):
        rows = idx[b * seqlen_q:(b + 1) * seqlen_q].astype(np.int64)    # [Sq, NHK, topk]
        valid = (rows >= 0) & (rows < seqlen_k)
        i = np.broadcast_to(np.arange(seqlen_q)[:, None, None], rows.shape)[valid]
        hk = np.broadcast_to(np.arange(nhk)[None, :, None], rows.shape)[valid]
        tok[b, hk, i, rows[valid]] = True
    return tok


def presence_to_csr(presence):
    """(q2k_row_ptr, q2k_col, k2q_row_ptr, k2q_col), all int32.

    ``presence`` is [B, H, nQB, nKB] (any integer/bool dtype, nonzero = kept).
    Q->K rows are (b, h, qb) in that order with ascending kb; K->Q rows are
    (b, h, kb) with ascending qb.
    """
    p = np.asarray(presence) != 0
    B, H, n_qb, n_kb = p.shape
    q_ptr = [0]
    q_col = []
    for b in range(B):
        for h in range(H):
            for qb in range(n_qb):
                cols = np.nonzero(p[b, h, qb, :])[0]
                q_col.extend(cols.tolist())
                q_ptr.append(len(q_col))
    k_ptr = [0]
    k_col = []
    for b in range(B):
        for h in range(H):
            for kb in range(n_kb):
                rows = np.nonzero(p[b, h, :, kb])[0]
                k_col.extend(rows.tolist())
                k_ptr.append(len(k_col))
    return (np.asarray(q_ptr, dtype=np.int32), np.asarray(q_col, dtype=np.int32),
            np.asarray(k_ptr, dtype=np.int32), np.asarray(k_col, dtype=np.int32))
