"""GPU parity of the attention forward (O and LSE) against the fp64 oracle
forward, on the same cases as the backward parity tests."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_close, bits_to_dev, dev_to_f64, gpu_mask, log
from tests.test_gpu_parity import CASES, get_case

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4          # relative; scores are exact fp32 sums of bf16 products


@pytest.mark.parametrize("name", list(CASES))
def test_attn_fwd_parity(name):
    import torch
    import index_sparse_attention_amd as isa
    c = get_case(name)
    d = c.data
    log(f"forward {name} [{c.label()}]")
    q, k, v = bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"])
    o, lse = isa.attn_fwd(q, k, v, mask=gpu_mask(c), causal=c.causal, softmax_scale=c.scale)
    torch.cuda.synchronize()
    heads = list(range(c.Hq)) if c.heads is None else list(c.heads)
    got_o = dev_to_f64(o)[:, :, heads, :]
    ref_o = d["o64"][:, :, heads, :]
    assert_close("o", got_o, ref_o)
    got_l = lse.cpu().numpy().astype(np.float64)[:, heads, :]
    ref_l = d["lse64"][:, heads, :]
    empty = np.isinf(ref_l)
    assert np.array_equal(np.isinf(got_l), empty), "rows with no kept key must have LSE = +inf"
    assert np.all(got_l[empty] > 0)
    if (~empty).any():
        err = np.abs(got_l[~empty] - ref_l[~empty]) / np.maximum(1.0, np.abs(ref_l[~empty]))
        log(f"  lse: max rel err {err.max():.3e}")
        assert err.max() <= LSE_TOL
    # rows with no kept key have O = 0
    assert np.all(got_o[:, :, :, :][np.broadcast_to(empty.transpose(0, 2, 1)[..., None], got_o.shape)] == 0)


def test_fwd_then_bwd_matches_oracle():
    """The GPU forward's O and LSE fed to the GPU backward give the oracle's
    gradients (the oracle backward from its own forward)."""
    import torch
    import index_sparse_attention_amd as isa
    from tests.gpu_helpers import oracle_grads
    c = get_case("block_h1_gqa_causal")
    d = c.data
    q, k, v, do = (bits_to_dev(d[n]) for n in ("q", "k", "v", "do"))
    m = gpu_mask(c)
    o, lse = isa.attn_fwd(q, k, v, mask=m, causal=c.causal, softmax_scale=c.scale)
    dq, dk, dv = isa.attn_bwd(q, k, v, o, do, lse, mask=m, causal=c.causal, softmax_scale=c.scale, algo="split")
    torch.cuda.synchronize()
    rq, rk, rv = oracle_grads(c)
    assert_close("dq", dev_to_f64(dq), rq)
    assert_close("dk", dev_to_f64(dk), rk)
    assert_close("dv", dev_to_f64(dv), rv)
