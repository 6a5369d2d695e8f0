"""Shared pieces of the GPU parity tests: seeded inputs, oracle references,
GPU calls through the C ABI, and the tolerance check.

Tolerance (per tensor): max|gpu - ref| <= 2e-2 * max|ref| + 1e-3, with the
reference from the fp64 oracle on the exact same bf16 inputs (O rounded to
bf16 and LSE rounded to fp32, as the GPU receives them).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import synth

REL_TOL = 2e-2
ABS_TOL = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def max_err(got: np.ndarray, ref: np.ndarray):
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    bound = REL_TOL * (float(np.abs(ref).max()) if ref.size else 0.0) + ABS_TOL
    return err, bound


def assert_close(name: str, got: np.ndarray, ref: np.ndarray):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err, bound = max_err(got, ref)
    log(f"  {name}: max|gpu-ref| = {err:.3e}  bound = {bound:.3e}")
    assert err <= bound, f"{name}: max|gpu-ref| = {err:.4e} > {bound:.4e}"


@dataclass
class Case:
    B: int
    Sq: int
    Sk: int
    Hq: int
    Hk: int
    Dqk: int
    Dv: int
    causal: bool = False
    mask: str = "dense"          # dense | block | index
    Hm: int = 0                  # block masks: mask heads (default Hq)
    keep: float = 0.5
    topk: int = 64
    seed: int = 0
    heads: list | None = None    # query heads with real O/LSE (others: LSE = +inf)
    token: bool = False          # index masks: token-exact (each query attends only its selected keys)
    data: dict = field(default_factory=dict)

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.Dqk)))

    def label(self):
        return (f"B{self.B} Sq{self.Sq} Sk{self.Sk} Hq{self.Hq} Hk{self.Hk} D{self.Dqk}/{self.Dv} "
                f"{'causal ' if self.causal else ''}{self.mask}{' token' if self.token else ''} seed{self.seed}")


def build_case(c: Case) -> Case:
    """Draw inputs, build the oracle's mask and forward outputs."""
    g = synth.seed_streams(c.seed)
    d = c.data
    d["q"] = synth.bf16_normal(g[0], (c.B, c.Sq, c.Hq, c.Dqk))
    d["k"] = synth.bf16_normal(g[1], (c.B, c.Sk, c.Hk, c.Dqk))
    d["v"] = synth.bf16_normal(g[2], (c.B, c.Sk, c.Hk, c.Dv))
    d["do"] = synth.bf16_normal(g[3], (c.B, c.Sq, c.Hq, c.Dv))
    n_qb, n_kb = -(-c.Sq // 128), -(-c.Sk // 128)
    if c.mask == "block":
        Hm = c.Hm or c.Hq
        d["presence"] = synth.block_mask(g[4], c.B, Hm, n_qb, n_kb, c.keep, force_diag=True)
        d["csr"] = oracle.presence_to_csr(d["presence"])
        d["omask"] = oracle.block_mask_from_csr(Hm, *d["csr"])
    elif c.mask == "index":
        d["indices"] = synth.topk_indices(g[5], c.B, c.Sq, c.Sk, c.Hk, c.topk, causal=True)
        d["presence"] = oracle.indices_to_presence(d["indices"], c.B, c.Sq, c.Sk)
        d["csr"] = oracle.presence_to_csr(d["presence"])
        tok = oracle.indices_to_token_mask(d["indices"], c.B, c.Sq, c.Sk) if c.token else None
        d["omask"] = oracle.block_mask_from_csr(c.Hk, *d["csr"], token=tok)
    else:
        d["omask"] = oracle.dense_mask()
    f = {k: oracle.bf16_to_f64(d[k]) for k in ("q", "k", "v", "do")}
    O, L = oracle.attn_fwd(f["q"], f["k"], f["v"], d["omask"], c.causal, c.scale, heads=c.heads)
    d["o64"], d["lse64"] = O, L
    d["o"] = oracle.round_to_bf16(O)
    d["lse"] = oracle.round_to_f32(L)
    return c


def oracle_grads(c: Case, order: str = "K"):
    d = c.data
    f = {k: oracle.bf16_to_f64(d[k]) for k in ("q", "k", "v", "do", "o")}
    return oracle.attn_bwd(f["q"], f["k"], f["v"], f["o"], f["do"], d["lse"].astype(np.float64),
                           d["omask"], c.causal, c.scale, order=order, heads=c.heads)


def gpu_mask(c: Case):
    """The GPU-built BlockMask for block/index cases (None for dense)."""
    import index_sparse_attention_amd as isa
    d = c.data
    if c.mask == "block":
        return isa.block_mask_to_csr(torch.from_numpy(d["presence"]).cuda())
    if c.mask == "index":
        return isa.index_to_block_sparse(torch.from_numpy(d["indices"]).cuda(), c.B, c.Sq, c.Sk, token_exact=c.token)
    return None


def csr_to_host(m, nnz=None):
    qp = m.q2k_row_ptr.cpu().numpy()
    kp = m.k2q_row_ptr.cpu().numpy()
    n = int(qp[-1]) if nnz is None else nnz
    return qp, m.q2k_col[:n].cpu().numpy(), kp, m.k2q_col[:int(kp[-1])].cpu().numpy()


def assert_csr_equal(got, ref):
    names = ("q2k_row_ptr", "q2k_col", "k2q_row_ptr", "k2q_col")
    for n, a, b in zip(names, got, ref):
        assert a.dtype == np.int32, n
        assert a.shape == b.shape and np.array_equal(a, b), f"{n} differs"


def run_gpu(c: Case, algo: str, mask=None, workspace_fill: int | None = None):
    import index_sparse_attention_amd as isa
    d = c.data
    q, k, v = bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"])
    o, do = bits_to_dev(d["o"]), bits_to_dev(d["do"])
    lse = torch.from_numpy(np.ascontiguousarray(d["lse"])).cuda()
    ws = None
    if workspace_fill is not None:
        # sized by the mask's kept blocks: SPLIT_DS gets exactly the dS tiles it needs
        if mask is not None:
            mask.nnz()
        need = isa.attn_bwd_workspace_bytes(c.B, c.Sq, c.Sk, c.Hq, c.Hk, c.Dqk, c.Dv, algo, mask=mask,
                                            causal=c.causal)
        ws = torch.full((max(need, 1),), workspace_fill, dtype=torch.uint8, device="cuda")
    dq, dk, dv = isa.attn_bwd(q, k, v, o, do, lse, mask=mask, causal=c.causal,
                              softmax_scale=c.scale, algo=algo, workspace=ws)
    torch.cuda.synchronize()
    return dev_to_f64(dq), dev_to_f64(dk), dev_to_f64(dv)
