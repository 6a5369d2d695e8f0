"""GPU parity of token-exact index masking (each query attends exactly the
keys its index row selects, not every key of a kept block): the converter's
token bits, the forward and both two-pass backward algorithms against the
fp64 oracle with its token term, for fixed-length and packed sequences."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (Case, assert_close, bits_to_dev, build_case, dev_to_f64, gpu_mask, log,
                               oracle_grads, run_gpu)

pytestmark = pytest.mark.gpu

CASES = {
    "tok_gqa_d128": Case(1, 640, 640, 4, 2, 128, 128, mask="index", topk=96, seed=51, token=True),
    "tok_gqa_causal_ragged": Case(1, 300, 420, 4, 1, 128, 128, causal=True, mask="index", topk=40, seed=52,
                                  token=True),
    "tok_mha_d64_b2": Case(2, 256, 384, 2, 2, 64, 64, mask="index", topk=24, seed=53, token=True),
    "tok_d192": Case(1, 384, 384, 2, 1, 192, 128, causal=True, mask="index", topk=64, seed=54, token=True),
}
_built = {}


def get(name):
    if name not in _built:
        _built[name] = build_case(CASES[name])
    return _built[name]


def test_token_bits_match_the_oracle():
    """Converter bits (both layouts) equal the oracle's token term."""
    c = get("tok_gqa_causal_ragged")
    m = gpu_mask(c)
    bits = m.token_bits.cpu().numpy().view(np.uint32)
    tok = oracle.indices_to_token_mask(c.data["indices"], c.B, c.Sq, c.Sk)
    B, H, n_qb, n_kb = c.B, c.Hk, m.n_qb, m.n_kb
    slots = bits[:B * H * n_qb * n_kb * 1024].reshape(B, H, n_qb, n_kb, 1024)
    row = np.unpackbits(slots[..., :512].reshape(B, H, n_qb, n_kb, 128, 4).view(np.uint8), axis=-1,
                        bitorder="little").reshape(B, H, n_qb, n_kb, 128, 128)
    key = np.unpackbits(slots[..., 512:].reshape(B, H, n_qb, n_kb, 128, 4).view(np.uint8), axis=-1,
                        bitorder="little").reshape(B, H, n_qb, n_kb, 128, 128)
    full = np.zeros((B, H, n_qb * 128, n_kb * 128), dtype=bool)
    full[:, :, :c.Sq, :c.Sk] = tok
    want = full.reshape(B, H, n_qb, 128, n_kb, 128).transpose(0, 1, 2, 4, 3, 5)
    assert np.array_equal(row.astype(bool), want)
    assert np.array_equal(key.astype(bool), want.transpose(0, 1, 2, 3, 5, 4))


@pytest.mark.parametrize("name", list(CASES))
def test_token_forward(name):
    import index_sparse_attention_amd as isa
    c = get(name)
    log(f"token forward {name} [{c.label()}]")
    d = c.data
    o, lse = isa.attn_fwd(bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"]), mask=gpu_mask(c),
                          causal=c.causal, softmax_scale=c.scale)
    torch.cuda.synchronize()
    assert_close("o", dev_to_f64(o), d["o64"])
    got, ref = lse.cpu().numpy().astype(np.float64), d["lse64"]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.abs(got[fin] - ref[fin]).max() / max(1.0, np.abs(ref[fin]).max()) < 1e-4


@pytest.mark.parametrize("algo", ["split", "split_ds"])
@pytest.mark.parametrize("name", list(CASES))
def test_token_backward(name, algo):
    c = get(name)
    log(f"token backward {name} algo={algo} [{c.label()}]")
    dq, dk, dv = run_gpu(c, algo, gpu_mask(c), workspace_fill=0xFF)
    rq, rk, rv = oracle_grads(c)
    assert_close("dq", dq, rq)
    assert_close("dk", dk, rk)
    assert_close("dv", dv, rv)


def test_token_mask_differs_from_block_mask():
    """The token term changes the result (the test above would not notice a
    kernel that ignores the bits if selected keys filled whole blocks)."""
    c = get("tok_gqa_d128")
    blk = Case(**{**c.__dict__, "token": False, "data": {}})
    blk = build_case(blk)
    rq_tok = oracle_grads(c)[0]
    rq_blk = oracle_grads(blk)[0]
    assert np.abs(rq_tok - rq_blk).max() > 10 * (2e-2 * np.abs(rq_tok).max() + 1e-3)


def test_token_varlen():
    """Token-exact bits of packed sequences: each sequence on its own."""
    import index_sparse_attention_amd as isa
    lens = [300, 128, 77]
    subs = [build_case(Case(1, L, L, 2, 1, 64, 64, causal=True, mask="index", topk=32, seed=60 + i, token=True))
            for i, L in enumerate(lens)]
    cat = lambda k: np.concatenate([s.data[k][0] if k != "indices" else s.data[k] for s in subs], axis=0)
    q, k, v, o, do, idx = (cat(x) for x in ("q", "k", "v", "o", "do", "indices"))
    B, M = len(lens), max(lens)
    lse = np.full((B, 2, M), np.inf, dtype=np.float32)
    for b, s in enumerate(subs):
        lse[b, :, :lens[b]] = s.data["lse"][0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    m = isa.index_to_block_sparse(torch.from_numpy(idx).cuda(), B, M, M, cu_seqlens_q=cu, cu_seqlens_k=cu,
                                  token_exact=True)
    for algo in ("split", "split_ds"):
        got = isa.attn_bwd(bits_to_dev(q), bits_to_dev(k), bits_to_dev(v), bits_to_dev(o), bits_to_dev(do),
                           torch.from_numpy(lse).cuda(), mask=m, causal=True, softmax_scale=subs[0].scale,
                           algo=algo, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=M, max_seqlen_k=M)
        torch.cuda.synchronize()
        refs = [oracle_grads(s) for s in subs]
        for i, n in enumerate(("dq", "dk", "dv")):
            assert_close(f"{algo} {n}", dev_to_f64(got[i]), np.concatenate([r[i][0] for r in refs], axis=0))
    ov, _ = isa.attn_fwd(bits_to_dev(q), bits_to_dev(k), bits_to_dev(v), mask=m, causal=True,
                         softmax_scale=subs[0].scale, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=M,
                         max_seqlen_k=M)
    torch.cuda.synchronize()
    assert_close("o", dev_to_f64(ov), np.concatenate([s.data["o64"][0] for s in subs], axis=0))
