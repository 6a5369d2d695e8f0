"""GPU parity at the five benchmark workloads' full sizes, in the launch
configuration the benchmark times.

The fp64 oracle cannot run the whole of the larger workloads in test time, so
a subset of query heads carries real forward outputs (O, LSE from the oracle
forward) and is checked element by element; every other head gets LSE = +inf
(no visible key: P = 0), which the backward must turn into exact zeros -- a
check that holds at any size and catches cross-head writes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import (Case, assert_close, assert_csr_equal, bits_to_dev, csr_to_host, dev_to_f64,
                               log)

pytestmark = pytest.mark.gpu

# workload -> query heads checked against the oracle (None = all)
CHECKED = {
    "dense_mha_s256_d64": None,
    "causal_gqa_s2k_d128": None,
    "blocksparse_mha_s8k_d128": [0, 13],
    "indexsparse_gqa_s16k_d128": [0, 1, 8],        # KV heads 0 and 1
    "causal_mha_s32k_d192": [5, 15],
}

_cache = {}


def workload_case(name):
    if name in _cache:
        return _cache[name]
    w = synth.WORKLOADS[name]
    log(f"building workload {name}")
    d = synth.make_workload_inputs(w)
    if w.mask == "block":
        d["csr"] = oracle.presence_to_csr(d["presence"])
        omask = oracle.block_mask_from_csr(w.mask_heads, *d["csr"])
    elif w.mask == "index":
        d["presence"] = oracle.indices_to_presence(d["indices"], w.batch, w.seqlen_q, w.seqlen_k)
        d["csr"] = oracle.presence_to_csr(d["presence"])
        omask = oracle.block_mask_from_csr(w.heads_k, *d["csr"])
    else:
        omask = oracle.dense_mask()
    heads = CHECKED[name]
    f = {k: oracle.bf16_to_f64(d[k]) for k in ("q", "k", "v", "do")}
    O, L = oracle.attn_fwd(f["q"], f["k"], f["v"], omask, w.causal, w.scale, heads=heads)
    d["o"] = oracle.round_to_bf16(O)
    d["lse"] = oracle.round_to_f32(L)
    del O
    log(f"oracle backward {name} heads={heads}")
    ref = oracle.attn_bwd(f["q"], f["k"], f["v"], oracle.bf16_to_f64(d["o"]), f["do"],
                          d["lse"].astype(np.float64), omask, w.causal, w.scale, heads=heads)
    _cache[name] = (w, d, ref)
    return _cache[name]


def gpu_mask(w, d):
    import index_sparse_attention_amd as isa
    if w.mask == "block":
        return isa.block_mask_to_csr(torch.from_numpy(d["presence"]).cuda())
    if w.mask == "index":
        return isa.index_to_block_sparse(torch.from_numpy(d["indices"]).cuda(), w.batch, w.seqlen_q,
                                         w.seqlen_k)
    return None


@pytest.mark.parametrize("algo", ["loopk", "loopq", "split", "split_ds"])
@pytest.mark.parametrize("name", list(CHECKED))
def test_workload_full_size(name, algo):
    import index_sparse_attention_amd as isa
    w, d, (rq, rk, rv) = workload_case(name)
    log(f"workload {name} algo={algo}")
    mask = gpu_mask(w, d)
    if mask is not None:
        assert_csr_equal(csr_to_host(mask), d["csr"])
    # the workspace is sized by the kept blocks (SPLIT_DS: exactly the dS tiles the mask needs)
    dq, dk, dv = isa.attn_bwd(bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"]),
                              bits_to_dev(d["o"]), bits_to_dev(d["do"]),
                              torch.from_numpy(d["lse"]).cuda(), mask=mask, causal=w.causal,
                              softmax_scale=w.scale, algo=algo)
    torch.cuda.synchronize()
    dq, dk, dv = dev_to_f64(dq), dev_to_f64(dk), dev_to_f64(dv)
    heads = CHECKED[name]
    if heads is None:
        assert_close("dq", dq, rq)
        assert_close("dk", dk, rk)
        assert_close("dv", dv, rv)
        return
    G = w.heads_q // w.heads_k
    kv = sorted({h // G for h in heads})
    other_q = [h for h in range(w.heads_q) if h not in heads]
    other_kv = [h for h in range(w.heads_k) if h not in kv]
    assert_close("dq[checked heads]", dq[:, :, heads], rq[:, :, heads])
    assert_close("dk[checked kv heads]", dk[:, :, kv], rk[:, :, kv])
    assert_close("dv[checked kv heads]", dv[:, :, kv], rv[:, :, kv])
    assert np.all(dq[:, :, other_q] == 0), "dq of LSE=+inf heads must be exactly zero"
    if other_kv:
        assert np.all(dk[:, :, other_kv] == 0) and np.all(dv[:, :, other_kv] == 0)
