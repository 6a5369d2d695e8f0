"""Python binding over libisattn.so: argument marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the tensors are not on a GPU, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _abi

ALGOS = {"loopk": _abi.ALGO_LOOPK, "loopq": _abi.ALGO_LOOPQ, "split": _abi.ALGO_SPLIT,
         "split_ds": _abi.ALGO_SPLIT_DS}
# "auto" takes SPLIT_DS when its dS store fits this fraction of the free device memory, else SPLIT
AUTO_FREE_FRACTION = 0.8


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _view(t: torch.Tensor, name: str) -> _abi.Tensor:
    if t.dim() == 3:                               # packed sequences: [total, heads, dim]
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError(f"{name}: expected [batch, seq, heads, dim], got shape {tuple(t.shape)}")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name}: expected bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    return _abi.Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _varlen(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k):
    """Packed-sequence arguments: (batch, max_q, max_k, Varlen) or None."""
    if cu_seqlens_q is None and cu_seqlens_k is None:
        return None
    for n, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if c is None or c.dtype != torch.int32 or c.dim() != 1 or not c.is_cuda or not c.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor [batch + 1]")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    if max_seqlen_q is None or max_seqlen_k is None:
        lq = (cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item() if cu_seqlens_q.numel() > 1 else 0
        lk = (cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item() if cu_seqlens_k.numel() > 1 else 0
        max_seqlen_q = int(lq) if max_seqlen_q is None else max_seqlen_q
        max_seqlen_k = int(lk) if max_seqlen_k is None else max_seqlen_k
    return (cu_seqlens_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k),
            _abi.Varlen(cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()))


@dataclass
class BlockMask:
    """Block-sparse mask as device CSR arrays (int32), 128x128 blocks.

    q2k: per (batch, mask head, query block) the ascending key blocks;
    k2q: per (batch, mask head, key block) the ascending query blocks;
    token_bits: optional token-exact bits (int32 [batch*heads*n_qb*n_kb*1024],
    the layout of isattn_mask_t.token_bits): inside a kept block a pair is
    attended only if its bit is set.
    nnz_host: the number of kept blocks when known on the host (SPLIT_DS
    sizes its dS store by it); None until ``nnz()`` reads it."""
    heads: int
    n_qb: int
    n_kb: int
    q2k_row_ptr: torch.Tensor
    q2k_col: torch.Tensor
    k2q_row_ptr: torch.Tensor
    k2q_col: torch.Tensor
    block_q: int = 128
    block_k: int = 128
    token_bits: torch.Tensor | None = None
    nnz_host: int | None = None

    def nnz(self) -> int:
        """Number of kept blocks (reads the last row pointer once: synchronises)."""
        if self.nnz_host is None:
            self.nnz_host = int(self.q2k_row_ptr[-1].item())
        return self.nnz_host

    def _abi(self) -> _abi.Mask:
        return _abi.Mask(_abi.MASK_BLOCK_CSR, self.block_q, self.block_k, self.heads,
                         self.q2k_row_ptr.data_ptr(), self.q2k_col.data_ptr(),
                         self.k2q_row_ptr.data_ptr(), self.k2q_col.data_ptr(),
                         self.token_bits.data_ptr() if self.token_bits is not None else None,
                         -1 if self.nnz_host is None else int(self.nnz_host))


_DENSE = lambda: _abi.Mask(_abi.MASK_DENSE, 128, 128, 0, None, None, None, None, None, -1)


class Timer:
    """Stage timer of isattn_attn_bwd_timed (preprocess, two main kernels, postprocess)."""

    def __init__(self, capacity: int = 256):
        lib = _abi.load()
        h = ctypes.c_void_p()
        _abi.check(lib.isattn_timer_create(capacity, ctypes.byref(h)), "isattn_timer_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def reset(self):
        _abi.check(_abi.load().isattn_timer_reset(self._h), "isattn_timer_reset")

    def read(self):
        """(n_calls, [pre, main_a, main_b, post] milliseconds summed over the calls)."""
        n = ctypes.c_int32()
        ms = (ctypes.c_float * 4)()
        _abi.check(_abi.load().isattn_timer_read(self._h, ctypes.byref(n), ms), "isattn_timer_read")
        return n.value, [ms[0], ms[1], ms[2], ms[3]]

    def close(self):
        if getattr(self, "_h", None) is not None:
            _abi.load().isattn_timer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def attn_bwd_workspace_bytes(batch, seqlen_q, seqlen_k, heads_q, heads_k, dim_qk, dim_v,
                             algo="split", mask: "BlockMask | None | str" = "any", causal: bool = False,
                             varlen: bool = False) -> int:
    """Workspace bytes of ``attn_bwd``.  ``mask="any"`` (default) sizes for
    any mask (SPLIT_DS: a dS tile for every block); None (dense) or a
    BlockMask sizes SPLIT_DS's dS store by the kept blocks (a BlockMask's
    ``nnz_host`` if set, else every block of every mask head)."""
    shape = _abi.Shape(batch, seqlen_q, seqlen_k, heads_q, heads_k, dim_qk, dim_v)
    lib = _abi.load()
    if isinstance(mask, str):
        return int(lib.isattn_attn_bwd_workspace_bytes(ctypes.byref(shape), ALGOS[algo]))
    m = mask._abi() if mask is not None else _DENSE()
    return int(lib.isattn_attn_bwd_workspace_bytes_mask(ctypes.byref(shape), ALGOS[algo], ctypes.byref(m),
                                                       int(bool(causal)), int(bool(varlen))))


def choose_algo(batch, seqlen_q, seqlen_k, heads_q, heads_k, dim_qk, dim_v, mask=None, causal=False,
                varlen=False, device=None) -> str:
    """SPLIT_DS (faster) when its workspace, with the dS store sized by the
    kept blocks, fits AUTO_FREE_FRACTION of the free device memory; SPLIT
    (a workspace of a few MiB) otherwise.  Reads a BlockMask's block count
    (one synchronisation) if it is not known yet."""
    if mask is not None:
        mask.nnz()
    need = attn_bwd_workspace_bytes(batch, seqlen_q, seqlen_k, heads_q, heads_k, dim_qk, dim_v, "split_ds",
                                    mask=mask, causal=causal, varlen=varlen)
    free, _ = torch.cuda.mem_get_info(device)
    return "split_ds" if need <= AUTO_FREE_FRACTION * free else "split"


def _dims(q, k, v, vl):
    """(B, Sq, Sk, Hq, Hk, Dqk, Dv) of fixed-length [B,S,H,D] tensors or of
    packed [total,H,D] tensors with their varlen tuple."""
    if vl is None:
        B, Sq, Hq, Dqk = q.shape
        return B, Sq, k.shape[1], Hq, k.shape[2], Dqk, v.shape[3]
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed sequences take q, k, v as [total_tokens, heads, dim]")
    return vl[0], vl[1], vl[2], q.shape[1], k.shape[1], q.shape[2], v.shape[2]


def attn_bwd(q, k, v, o, do, lse, mask: BlockMask | None = None, causal: bool = False,
             softmax_scale: float | None = None, algo: str = "auto", dq=None, dk=None, dv=None,
             workspace: torch.Tensor | None = None, stream=None, timer: Timer | None = None,
             cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None):
    """Attention backward on the GPU.  Returns (dq, dk, dv) as bf16 tensors.

    q [B,Sq,Hq,Dqk], k [B,Sk,Hk,Dqk], v [B,Sk,Hk,Dv], o/do [B,Sq,Hq,Dv] bf16;
    lse fp32 [B,Hq,Sq] (natural log).  ``mask`` None = dense.  ``causal``
    adds the bottom-right causal term.  Outputs are allocated when not given.
    ``algo``: "auto" (default: "split_ds" when its workspace fits the free
    device memory, else "split"), "split" (two atomic-free passes, a
    workspace of a few MiB), "split_ds" (the dK/dV pass stores dS for the dQ
    pass: faster, 32 KiB of workspace per kept block and query head), "loopk"
    or "loopq" (the pages' loop orders with fp32 atomics).  A workspace
    allocated here for "split_ds" is sized by the mask's kept blocks (a
    BlockMask's count is read once if not known: one synchronisation).
    Packed sequences: pass int32 ``cu_seqlens_q`` / ``cu_seqlens_k`` [B + 1]
    and q, k, v, o, do as [total_tokens, heads, dim]; lse is then
    [B, Hq, max_seqlen_q] (the longest lengths are computed when not given,
    which synchronises); "split" and "split_ds" only.
    """
    lib = _abi.load()
    vl = _varlen(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    B, Sq, Sk, Hq, Hk, Dqk, Dv = _dims(q, k, v, vl)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    shape = _abi.Shape(B, Sq, Sk, Hq, Hk, Dqk, Dv)
    if algo == "auto":
        algo = choose_algo(B, Sq, Sk, Hq, Hk, Dqk, Dv, mask=mask, causal=causal, varlen=vl is not None,
                           device=q.device)
    a = ALGOS[algo]
    if workspace is None:
        if algo == "split_ds" and mask is not None:
            mask.nnz()
        need = attn_bwd_workspace_bytes(B, Sq, Sk, Hq, Hk, Dqk, Dv, algo, mask=mask, causal=causal,
                                        varlen=vl is not None)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    views = [_view(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"),
                                      (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    m = mask._abi() if mask is not None else _DENSE()
    args = [ctypes.byref(x) for x in views[:5]] + [
        lse.data_ptr(), ctypes.byref(m), int(bool(causal)), float(softmax_scale)] + [
        ctypes.byref(x) for x in views[5:]] + [a, workspace.data_ptr(), workspace.numel(),
                                               _stream_ptr(stream)]
    if vl is not None:
        if timer is not None:
            raise ValueError("stage timing is not available for packed sequences")
        _abi.check(lib.isattn_attn_bwd_varlen(ctypes.byref(shape), ctypes.byref(vl[3]), *args),
                   "isattn_attn_bwd_varlen")
    elif timer is None:
        _abi.check(lib.isattn_attn_bwd(ctypes.byref(shape), *args), "isattn_attn_bwd")
    else:
        _abi.check(lib.isattn_attn_bwd_timed(ctypes.byref(shape), *args, timer.handle), "isattn_attn_bwd_timed")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, mask: BlockMask | None = None, causal: bool = False,
                     softmax_scale: float | None = None, stream=None):
    """``attn_bwd`` with algo "split" through isattn_attn_bwd_noalloc: the
    library allocates nothing (its workspace is a static 64 MiB device array
    per GPU) and this wrapper allocates nothing either -- the caller passes
    dq, dk, dv.  Calls that overlap on one GPU race on the shared scratch.
    Returns (dq, dk, dv)."""
    lib = _abi.load()
    B, Sq, Sk, Hq, Hk, Dqk, Dv = _dims(q, k, v, None)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    shape = _abi.Shape(B, Sq, Sk, Hq, Hk, Dqk, Dv)
    views = [_view(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"),
                                      (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    m = mask._abi() if mask is not None else _DENSE()
    args = [ctypes.byref(x) for x in views[:5]] + [
        lse.data_ptr(), ctypes.byref(m), int(bool(causal)), float(softmax_scale)] + [
        ctypes.byref(x) for x in views[5:]] + [_stream_ptr(stream)]
    _abi.check(lib.isattn_attn_bwd_noalloc(ctypes.byref(shape), *args), "isattn_attn_bwd_noalloc")
    return dq, dk, dv


def attn_fwd(q, k, v, mask: BlockMask | None = None, causal: bool = False, softmax_scale: float | None = None,
             o=None, lse=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
             max_seqlen_k=None):
    """Attention forward on the GPU.  Returns (o bf16 [B,Sq,Hq,Dv], lse fp32
    [B,Hq,Sq], natural log, +inf for a row with no kept key).  Same mask,
    causal and packed-sequence conventions as ``attn_bwd`` (packed: o is
    [total_q, Hq, Dv]); outputs are allocated when not given.
    """
    lib = _abi.load()
    vl = _varlen(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    B, Sq, Sk, Hq, Hk, Dqk, Dv = _dims(q, k, v, vl)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if o is None:
        oshape = (B, Sq, Hq, Dv) if vl is None else (q.shape[0], Hq, Dv)
        o = torch.empty(oshape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.full((B, Hq, Sq), float("inf"), dtype=torch.float32, device=q.device) if vl is not None \
            else torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    shape = _abi.Shape(B, Sq, Sk, Hq, Hk, Dqk, Dv)
    vq, vk, vv, vo = (_view(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")))
    m = mask._abi() if mask is not None else _DENSE()
    args = [ctypes.byref(vq), ctypes.byref(vk), ctypes.byref(vv), ctypes.byref(m), int(bool(causal)),
            float(softmax_scale), ctypes.byref(vo), lse.data_ptr(), _stream_ptr(stream)]
    if vl is not None:
        _abi.check(lib.isattn_attn_fwd_varlen(ctypes.byref(shape), ctypes.byref(vl[3]), *args),
                   "isattn_attn_fwd_varlen")
    else:
        _abi.check(lib.isattn_attn_fwd(ctypes.byref(shape), *args), "isattn_attn_fwd")
    return o, lse


def topk_select(scores: torch.Tensor, topk: int, starts: torch.Tensor | None = None,
                ends: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Top-k positions of each fp32 score row (GPU): int32 [rows, topk],
    highest score first (ties: smaller position first), -1 padded.  Rows may
    be limited to [starts[r], ends[r]) (int32 [rows] each)."""
    lib = _abi.load()
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1 or not scores.is_cuda:
        raise ValueError("scores must be a float32 GPU tensor [rows, n] with contiguous rows")
    rows, n = scores.shape
    if (starts is None) != (ends is None):
        raise ValueError("give both starts and ends, or neither")
    for t in (starts, ends):
        if t is not None and (t.dtype != torch.int32 or t.numel() != rows or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("starts / ends must be contiguous int32 GPU tensors [rows]")
    out = torch.empty((rows, topk), dtype=torch.int32, device=scores.device) if out is None else out
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, topk) or not out.is_contiguous():
        raise ValueError("out must be contiguous int32 [rows, topk]")
    _abi.check(lib.isattn_topk_select(scores.data_ptr(), scores.stride(0), rows, n,
                                      starts.data_ptr() if starts is not None else None,
                                      ends.data_ptr() if ends is not None else None, topk, out.data_ptr(),
                                      _stream_ptr(stream)), "isattn_topk_select")
    return out


def _csr_buffers(rows_q, rows_k, nnz_max, device):
    i32 = dict(dtype=torch.int32, device=device)
    return (torch.empty(rows_q + 1, **i32), torch.empty(max(nnz_max, 1), **i32),
            torch.empty(rows_k + 1, **i32), torch.empty(max(nnz_max, 1), **i32))


def index_to_block_sparse(indices: torch.Tensor, batch: int, seqlen_q: int, seqlen_k: int,
                          block_q: int = 128, block_k: int = 128, stream=None, cu_seqlens_q=None,
                          cu_seqlens_k=None, token_exact: bool = False) -> BlockMask:
    """int32 indices [batch*seqlen_q, nhk, topk] -> BlockMask with heads = nhk.
    Packed sequences: give ``cu_seqlens_q`` / ``cu_seqlens_k`` (int32 [batch
    + 1]); indices are then [total_q, nhk, topk] and seqlen_q / seqlen_k the
    longest lengths.  ``token_exact``: also build the token bits, so that each
    query attends exactly its selected keys (else every pair of a kept block)."""
    lib = _abi.load()
    if indices.dtype != torch.int32 or indices.dim() != 3 or not indices.is_contiguous():
        raise ValueError("indices must be contiguous int32 [batch*seqlen_q, nhk, topk]")
    if not indices.is_cuda:
        raise ValueError("indices must be a GPU tensor")
    nhk, topk = indices.shape[1], indices.shape[2]
    n_qb, n_kb = -(-seqlen_q // block_q), -(-seqlen_k // block_k)
    nnz_max = batch * nhk * n_qb * n_kb
    qp, qc, kp, kc = _csr_buffers(batch * nhk * n_qb, batch * nhk * n_kb, nnz_max, indices.device)
    ws_bytes = int(lib.isattn_index_to_block_sparse_workspace_bytes(batch, seqlen_q, seqlen_k, nhk,
                                                                    block_q, block_k))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=indices.device)
    outs = (qp.data_ptr(), qc.data_ptr(), kp.data_ptr(), kc.data_ptr(), qc.numel(), ws.data_ptr(), ws.numel(),
            _stream_ptr(stream))
    if cu_seqlens_q is not None or cu_seqlens_k is not None:
        vl = _varlen(cu_seqlens_q, cu_seqlens_k, seqlen_q, seqlen_k)
        if vl[0] != batch:
            raise ValueError("cu_seqlens must have batch + 1 entries")
        _abi.check(lib.isattn_index_to_block_sparse_varlen(
            indices.data_ptr(), batch, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), seqlen_q, seqlen_k,
            nhk, topk, block_q, block_k, *outs), "isattn_index_to_block_sparse_varlen")
    else:
        _abi.check(lib.isattn_index_to_block_sparse(
            indices.data_ptr(), batch, seqlen_q, seqlen_k, nhk, topk, block_q, block_k, *outs),
            "isattn_index_to_block_sparse")
    bits = None
    if token_exact:
        if block_q != 128 or block_k != 128:
            raise ValueError("token-exact bits use 128 x 128 blocks")
        bits = torch.empty(max(batch * nhk * n_qb * n_kb * 1024, 4), dtype=torch.int32, device=indices.device)
        _abi.check(lib.isattn_index_to_token_bits(
            indices.data_ptr(), batch, seqlen_q, seqlen_k, nhk, topk,
            cu_seqlens_q.data_ptr() if cu_seqlens_q is not None else None,
            cu_seqlens_k.data_ptr() if cu_seqlens_k is not None else None,
            bits.data_ptr(), bits.numel(), _stream_ptr(stream)), "isattn_index_to_token_bits")
    return BlockMask(nhk, n_qb, n_kb, qp, qc, kp, kc, block_q, block_k, bits)


def block_mask_to_csr(presence: torch.Tensor, block_q: int = 128, block_k: int = 128,
                      stream=None) -> BlockMask:
    """uint8 presence [batch, heads, n_qb, n_kb] (nonzero = kept) -> BlockMask."""
    lib = _abi.load()
    if presence.dtype != torch.uint8 or presence.dim() != 4 or not presence.is_contiguous():
        raise ValueError("presence must be contiguous uint8 [batch, heads, n_qb, n_kb]")
    if not presence.is_cuda:
        raise ValueError("presence must be a GPU tensor")
    B, H, n_qb, n_kb = presence.shape
    nnz_max = B * H * n_qb * n_kb
    qp, qc, kp, kc = _csr_buffers(B * H * n_qb, B * H * n_kb, nnz_max, presence.device)
    ws_bytes = int(lib.isattn_block_mask_to_csr_workspace_bytes(B, H, n_qb, n_kb))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=presence.device)
    _abi.check(lib.isattn_block_mask_to_csr(
        presence.data_ptr(), B, H, n_qb, n_kb, qp.data_ptr(), qc.data_ptr(), kp.data_ptr(),
        kc.data_ptr(), qc.numel(), ws.data_ptr(), ws.numel(), _stream_ptr(stream)),
        "isattn_block_mask_to_csr")
    return BlockMask(H, n_qb, n_kb, qp, qc, kp, kc, block_q, block_k)
