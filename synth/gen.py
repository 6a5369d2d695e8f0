"""Seeded generators for the five attention-backward workloads.

Every tensor is produced from ``numpy.random.SeedSequence(seed).spawn(6)``;
stream 0..5 feed Q, K, V, dO, the block mask and the token indices.  bf16
tensors are returned as ``uint16`` bit patterns (round-to-nearest-even from
float32 normals), so a consumer can reinterpret them without any conversion
ambiguity.

The workload shapes follow the pages' correctness runs (MagiAttention PR #334,
"correctness verification" tables: D=128, MHA and GQA 8/2, block sparsity
0.5-0.75, top-k 256) scaled up to long sequences, plus the asymmetric 192/128
head dims of MagiAttention PR #331 (Summary).  The index lists mimic the DSA
indexer output described in xtuner PR #2096 (Main Changes, item 1): int32,
one row per query token, ``-1`` where a row has fewer valid positions than
top-k, entries ordered by score rather than by position.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np


# --------------------------------------------------------------------------
# bit-level bf16
# --------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 ~ N(0, std^2) as uint16 bits (float32 draw, then RNE to bf16)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits_from_f32(x)


def seed_streams(seed: int, n: int = 6):
    """Independent generators for Q, K, V, dO, mask, indices."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


# --------------------------------------------------------------------------
# masks and indices
# --------------------------------------------------------------------------
def block_mask(rng: np.random.Generator, batch: int, heads: int, n_qb: int, n_kb: int,
               keep_prob: float, force_diag: bool = True) -> np.ndarray:
    """uint8 presence [batch, heads, n_qb, n_kb]: each block kept with ``keep_prob``,
    independently; the diagonal block (qb == kb) forced on when ``force_diag``."""
    m = (rng.random((batch, heads, n_qb, n_kb)) < keep_prob).astype(np.uint8)
    if force_diag:
        d = np.arange(min(n_qb, n_kb))
        m[:, :, d, d] = 1
    return m


def topk_indices(rng: np.random.Generator, batch: int, seqlen_q: int, seqlen_k: int,
                 nhk: int, topk: int, causal: bool = True, chunk: int = 512) -> np.ndarray:
    """int32 [batch*seqlen_q, nhk, topk] token indices.

    For query row i and each KV head, ``topk`` positions are drawn uniformly
    without replacement from the valid range ([0, i + seqlen_k - seqlen_q] when
    ``causal``, else [0, seqlen_k)).  Rows with fewer valid positions keep all
    of them and pad the rest with -1.  Entries are listed in the order of the
    random draw key, i.e. not sorted by position.
    """
    out = np.empty((batch * seqlen_q, nhk, topk), dtype=np.int32)
    pos = np.arange(seqlen_k, dtype=np.int64)
    kk = min(topk, seqlen_k)
    for b in range(batch):
        for r0 in range(0, seqlen_q, chunk):
            r1 = min(seqlen_q, r0 + chunk)
            keys = rng.random((r1 - r0, nhk, seqlen_k))
            if causal:
                last = np.arange(r0, r1, dtype=np.int64) + (seqlen_k - seqlen_q)
                invalid = pos[None, :] > last[:, None]          # [rows, Sk]
                keys[np.broadcast_to(invalid[:, None, :], keys.shape)] = np.inf
            if kk < seqlen_k:
                sel = np.argpartition(keys, kk - 1, axis=-1)[..., :kk]
            else:
                sel = np.broadcast_to(pos, keys.shape).copy()
            kv = np.take_along_axis(keys, sel, axis=-1)
            order = np.argsort(kv, axis=-1, kind="stable")
            sel = np.take_along_axis(sel, order, axis=-1)
            kv = np.take_along_axis(kv, order, axis=-1)
            sel = sel.astype(np.int32)
            sel[np.isinf(kv)] = -1
            blk = out[b * seqlen_q + r0: b * seqlen_q + r1]
            blk[..., :kk] = sel
            if kk < topk:
                blk[..., kk:] = -1
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_k: int
    seqlen_q: int
    seqlen_k: int
    dim_qk: int
    dim_v: int
    causal: bool
    mask: str                 # "dense" | "block" | "index"
    keep_prob: float = 1.0    # block masks
    topk: int = 0             # index masks
    block: int = 128
    seed: int = 0

    @property
    def scale(self) -> float:
        """float32 value of 1/sqrt(dim_qk), returned as a Python float."""
        return float(np.float32(1.0 / math.sqrt(self.dim_qk)))

    @property
    def n_qb(self) -> int:
        return -(-self.seqlen_q // self.block)

    @property
    def n_kb(self) -> int:
        return -(-self.seqlen_k // self.block)

    @property
    def mask_heads(self) -> int:
        if self.mask == "block":
            return self.heads_q
        if self.mask == "index":
            return self.heads_k
        return 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # dense MHA, non-causal, short and narrow
    "dense_mha_s256_d64": Workload("dense_mha_s256_d64", 1, 2, 2, 256, 256, 64, 64,
                                   False, "dense", seed=1),
    # dense causal GQA 8/2 (bottom-right causal)
    "causal_gqa_s2k_d128": Workload("causal_gqa_s2k_d128", 2, 8, 2, 2048, 2048, 128, 128,
                                    True, "dense", seed=2),
    # 128x128 block-sparse MHA, each block kept with p=0.25, diagonal forced
    "blocksparse_mha_s8k_d128": Workload("blocksparse_mha_s8k_d128", 2, 16, 16, 8192, 8192,
                                         128, 128, False, "block", keep_prob=0.25, seed=3),
    # top-2048 token indices per query and KV head, converted to 128x128 blocks
    "indexsparse_gqa_s16k_d128": Workload("indexsparse_gqa_s16k_d128", 1, 16, 2, 16384, 16384,
                                          128, 128, False, "index", topk=2048, seed=4),
    # causal MHA with QK head dim 192 and V head dim 128
    "causal_mha_s32k_d192": Workload("causal_mha_s32k_d192", 1, 16, 16, 32768, 32768,
                                     192, 128, True, "dense", seed=5),
}


def make_workload_inputs(w: Workload, seed: int | None = None, want=("q", "k", "v", "do", "mask")):
    """Draw the random inputs of workload ``w``.

    Returns a dict with uint16 bf16 bits for q [B,Sq,Hq,Dqk], k [B,Sk,Hk,Dqk],
    v [B,Sk,Hk,Dv], do [B,Sq,Hq,Dv]; ``presence`` (uint8 [B,Hm,nQB,nKB]) for
    block masks; ``indices`` (int32 [B*Sq,Hk,topk]) for index masks.
    """
    s = w.seed if seed is None else seed
    g = seed_streams(s)
    out = {}
    if "q" in want:
        out["q"] = bf16_normal(g[0], (w.batch, w.seqlen_q, w.heads_q, w.dim_qk))
    if "k" in want:
        out["k"] = bf16_normal(g[1], (w.batch, w.seqlen_k, w.heads_k, w.dim_qk))
    if "v" in want:
        out["v"] = bf16_normal(g[2], (w.batch, w.seqlen_k, w.heads_k, w.dim_v))
    if "do" in want:
        out["do"] = bf16_normal(g[3], (w.batch, w.seqlen_q, w.heads_q, w.dim_v))
    if "mask" in want:
        if w.mask == "block":
            out["presence"] = block_mask(g[4], w.batch, w.mask_heads, w.n_qb, w.n_kb,
                                         w.keep_prob, force_diag=True)
        elif w.mask == "index":
            out["indices"] = topk_indices(g[5], w.batch, w.seqlen_q, w.seqlen_k,
                                          w.heads_k, w.topk, causal=True)
    return out
