"""GPU parity for packed variable-length sequences (cu_seqlens): forward and
the two-pass backward algorithms against the fp64 oracle applied to each
sequence on its own, the index converter's CSR against the oracle's per
sequence presence, and equality with the fixed-length path when every
sequence has the same length."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (Case, assert_close, assert_csr_equal, bits_to_dev, build_case, csr_to_host,
                               dev_to_f64, log, oracle_grads)

pytestmark = pytest.mark.gpu


@dataclass
class VarlenCase:
    lens_q: list
    lens_k: list
    Hq: int
    Hk: int
    Dqk: int
    Dv: int
    causal: bool = False
    mask: str = "dense"          # dense | block | index
    Hm: int = 0
    keep: float = 0.5
    topk: int = 48
    seed: int = 0
    data: dict = field(default_factory=dict)

    @property
    def B(self):
        return len(self.lens_q)

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.Dqk)))


CASES = {
    "dense_gqa_mixed": VarlenCase([130, 256, 1], [200, 384, 64], 4, 2, 128, 128, seed=31),
    "causal_mixed_d64": VarlenCase([300, 128, 77], [200, 128, 300], 2, 2, 64, 64, causal=True, seed=32),
    "block_mixed": VarlenCase([520, 256, 129], [520, 300, 129], 2, 2, 128, 128, mask="block", keep=0.4, seed=33),
    "block_gqa_causal": VarlenCase([384, 130], [384, 257], 4, 2, 128, 128, causal=True, mask="block", Hm=1,
                                   keep=0.5, seed=34),
    "index_gqa": VarlenCase([384, 200, 256], [384, 200, 256], 4, 2, 64, 64, mask="index", topk=40, seed=35),
    "causal_d192": VarlenCase([257, 130], [257, 300], 2, 1, 192, 128, causal=True, seed=36),
    "empty_sequences": VarlenCase([0, 130, 64], [100, 0, 64], 2, 2, 64, 64, seed=37),
}

_built = {}


def _empty_sub(vc, Sq, Sk):
    """A sequence with no queries or no keys: the oracle's results written out
    (no attended pair: O = 0, LSE = +inf, zero gradients)."""
    z = lambda *s: np.zeros(s, dtype=np.uint16)
    d = {"q": z(1, Sq, vc.Hq, vc.Dqk), "k": z(1, Sk, vc.Hk, vc.Dqk), "v": z(1, Sk, vc.Hk, vc.Dv),
         "do": z(1, Sq, vc.Hq, vc.Dv), "o": z(1, Sq, vc.Hq, vc.Dv),
         "o64": np.zeros((1, Sq, vc.Hq, vc.Dv)), "lse64": np.full((1, vc.Hq, Sq), np.inf),
         "lse": np.full((1, vc.Hq, Sq), np.inf, dtype=np.float32)}
    grads = (np.zeros((1, Sq, vc.Hq, vc.Dqk)), np.zeros((1, Sk, vc.Hk, vc.Dqk)), np.zeros((1, Sk, vc.Hk, vc.Dv)))
    return d, grads


def build(name):
    """Per-sequence oracle cases packed along the token dimension."""
    if name in _built:
        return _built[name]
    vc = CASES[name]
    subs = []
    for b, (Sq, Sk) in enumerate(zip(vc.lens_q, vc.lens_k)):
        if Sq == 0 or Sk == 0:
            subs.append(_empty_sub(vc, Sq, Sk) + (None,))
            continue
        c = build_case(Case(1, Sq, Sk, vc.Hq, vc.Hk, vc.Dqk, vc.Dv, causal=vc.causal, mask=vc.mask, Hm=vc.Hm,
                            keep=vc.keep, topk=vc.topk, seed=vc.seed * 100 + b))
        subs.append((c.data, oracle_grads(c), c))
    B, Sqm, Skm = vc.B, max(vc.lens_q), max(vc.lens_k)
    n_qb, n_kb = -(-Sqm // 128), -(-Skm // 128)
    d = vc.data
    cat = lambda key: np.concatenate([s[0][key][0] for s in subs], axis=0)
    for key in ("q", "k", "v", "do", "o"):
        d[key] = cat(key)
    d["o64"] = np.concatenate([s[0]["o64"][0] for s in subs], axis=0)
    d["lse"] = np.full((B, vc.Hq, Sqm), np.inf, dtype=np.float32)
    d["lse64"] = np.full((B, vc.Hq, Sqm), np.inf)
    for b, s in enumerate(subs):
        d["lse"][b, :, :vc.lens_q[b]] = s[0]["lse"][0]
        d["lse64"][b, :, :vc.lens_q[b]] = s[0]["lse64"][0]
    d["grads"] = tuple(np.concatenate([s[1][i][0] for s in subs], axis=0) for i in range(3))
    d["cu_q"] = np.concatenate([[0], np.cumsum(vc.lens_q)]).astype(np.int32)
    d["cu_k"] = np.concatenate([[0], np.cumsum(vc.lens_k)]).astype(np.int32)
    if vc.mask in ("block", "index"):
        Hm = (vc.Hm or vc.Hq) if vc.mask == "block" else vc.Hk
        pres = np.zeros((B, Hm, n_qb, n_kb), dtype=np.uint8)
        for b, s in enumerate(subs):
            if s[2] is not None:
                p = s[0]["presence"][0]
                pres[b, :, :p.shape[1], :p.shape[2]] = p
        d["presence"] = pres
        d["csr"] = oracle.presence_to_csr(pres)
    if vc.mask == "index":
        d["indices"] = np.concatenate([s[0]["indices"] for s in subs], axis=0)
    _built[name] = vc
    return vc


def gpu_mask(vc):
    import index_sparse_attention_amd as isa
    d = vc.data
    if vc.mask == "block":
        return isa.block_mask_to_csr(torch.from_numpy(d["presence"]).cuda())
    if vc.mask == "index":
        return isa.index_to_block_sparse(torch.from_numpy(d["indices"]).cuda(), vc.B, max(vc.lens_q),
                                         max(vc.lens_k), cu_seqlens_q=torch.from_numpy(d["cu_q"]).cuda(),
                                         cu_seqlens_k=torch.from_numpy(d["cu_k"]).cuda())
    return None


def cu(vc):
    return (torch.from_numpy(vc.data["cu_q"]).cuda(), torch.from_numpy(vc.data["cu_k"]).cuda())


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_forward(name):
    import index_sparse_attention_amd as isa
    vc = build(name)
    log(f"varlen forward {name}: lens_q {vc.lens_q} lens_k {vc.lens_k}")
    d = vc.data
    mask = gpu_mask(vc)
    if mask is not None:
        assert_csr_equal(csr_to_host(mask), d["csr"])
    cq, ck = cu(vc)
    o, lse = isa.attn_fwd(bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"]), mask=mask,
                          causal=vc.causal, softmax_scale=vc.scale, cu_seqlens_q=cq, cu_seqlens_k=ck,
                          max_seqlen_q=max(vc.lens_q), max_seqlen_k=max(vc.lens_k))
    torch.cuda.synchronize()
    assert_close("o", dev_to_f64(o), d["o64"])
    got = lse.cpu().numpy().astype(np.float64)
    for b, Sq in enumerate(vc.lens_q):
        g, r = got[b, :, :Sq], d["lse64"][b, :, :Sq]
        fin = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), fin), f"sequence {b}: +inf rows differ"
        if fin.any():
            err = np.abs(g[fin] - r[fin]).max() / max(1.0, np.abs(r[fin]).max())
            assert err < 1e-4, f"sequence {b}: lse rel err {err}"


@pytest.mark.parametrize("algo", ["split", "split_ds"])
@pytest.mark.parametrize("name", list(CASES))
def test_varlen_backward(name, algo):
    import index_sparse_attention_amd as isa
    vc = build(name)
    log(f"varlen backward {name} algo={algo}: lens_q {vc.lens_q} lens_k {vc.lens_k}")
    d = vc.data
    mask = gpu_mask(vc)
    cq, ck = cu(vc)
    need = isa.attn_bwd_workspace_bytes(vc.B, max(vc.lens_q), max(vc.lens_k), vc.Hq, vc.Hk, vc.Dqk, vc.Dv, algo)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes: must not leak
    dq, dk, dv = isa.attn_bwd(bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"]), bits_to_dev(d["o"]),
                              bits_to_dev(d["do"]), torch.from_numpy(d["lse"]).cuda(), mask=mask,
                              causal=vc.causal, softmax_scale=vc.scale, algo=algo, workspace=ws,
                              cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=max(vc.lens_q),
                              max_seqlen_k=max(vc.lens_k))
    torch.cuda.synchronize()
    for n, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), d["grads"]):
        assert_close(n, dev_to_f64(g), r)


@pytest.mark.parametrize("algo", ["split", "split_ds"])
@pytest.mark.parametrize("mask_kind", ["dense_causal", "index"])
def test_varlen_equal_lengths_match_fixed(algo, mask_kind):
    """Packed sequences of equal length go through the same kernels with the
    same arithmetic as the fixed-length batch: bit-identical results."""
    import index_sparse_attention_amd as isa
    if mask_kind == "index":
        c = build_case(Case(2, 256, 320, 4, 2, 128, 128, mask="index", topk=40, seed=38))
    else:
        c = build_case(Case(2, 256, 320, 4, 2, 128, 128, causal=True, seed=39))
    log(f"varlen == fixed {mask_kind} {algo}")
    d = c.data
    q, k, v, o, do = (bits_to_dev(d[x]) for x in ("q", "k", "v", "o", "do"))
    lse = torch.from_numpy(np.ascontiguousarray(d["lse"])).cuda()
    cq = torch.tensor([0, 256, 512], dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, 320, 640], dtype=torch.int32, device="cuda")
    if mask_kind == "index":
        idx = torch.from_numpy(d["indices"]).cuda()
        m_fix = isa.index_to_block_sparse(idx, 2, 256, 320)
        m_var = isa.index_to_block_sparse(idx, 2, 256, 320, cu_seqlens_q=cq, cu_seqlens_k=ck)
        for a, b in zip(csr_to_host(m_fix), csr_to_host(m_var)):
            assert np.array_equal(a, b)
    else:
        m_fix = m_var = None
    pk = lambda t: t.reshape(-1, t.shape[2], t.shape[3])
    fix = isa.attn_bwd(q, k, v, o, do, lse, mask=m_fix, causal=c.causal, softmax_scale=c.scale, algo=algo)
    var = isa.attn_bwd(pk(q), pk(k), pk(v), pk(o), pk(do), lse, mask=m_var, causal=c.causal,
                       softmax_scale=c.scale, algo=algo, cu_seqlens_q=cq, cu_seqlens_k=ck,
                       max_seqlen_q=256, max_seqlen_k=320)
    for n, x, y in zip(("dq", "dk", "dv"), fix, var):
        assert torch.equal(pk(x), y), f"{n} differs"
    of, lf = isa.attn_fwd(q, k, v, mask=m_fix, causal=c.causal, softmax_scale=c.scale)
    ov, lv = isa.attn_fwd(pk(q), pk(k), pk(v), mask=m_var, causal=c.causal, softmax_scale=c.scale,
                          cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=256, max_seqlen_k=320)
    torch.cuda.synchronize()
    assert torch.equal(pk(of), ov) and torch.equal(lf, lv)
