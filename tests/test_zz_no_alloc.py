"""isattn_attn_bwd_noalloc, the entry point that allocates nothing (its
workspace is the library's static per-GPU scratch), against the existing
entry point isattn_attn_bwd with algo SPLIT on the same inputs, on two calls
in a row -- the second smaller, so it runs over what the first left in the
scratch -- and against the fp64 oracle, at the usual tolerance.  Where the
existing entry point also runs its dK/dV pass one workgroup per item (512 or
more items), the two must agree bit for bit; with fewer items it cuts items
into parts and sums fp32 partials, so only the tolerance applies."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import (Case, assert_close, bits_to_dev, build_case, dev_to_f64, gpu_mask, log,
                               oracle_grads)

pytestmark = pytest.mark.gpu

CALLS = [
    # larger first: 512+ dK/dV items (no part mode in either entry point), block-sparse GQA
    ("block_gqa_many_items", Case(2, 256, 256, 256, 128, 64, 64, mask="block", Hm=128, keep=0.5, seed=31), True),
    # then smaller: ragged causal GQA with few items (the existing entry point uses part mode)
    ("causal_gqa_ragged", Case(1, 200, 333, 4, 2, 128, 128, causal=True, seed=32), False),
]


def run_both(c):
    import index_sparse_attention_amd as isa
    d = c.data
    q, k, v = bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"])
    o, do = bits_to_dev(d["o"]), bits_to_dev(d["do"])
    lse = torch.from_numpy(np.ascontiguousarray(d["lse"])).cuda()
    mask = gpu_mask(c)
    ref = isa.attn_bwd(q, k, v, o, do, lse, mask=mask, causal=c.causal, softmax_scale=c.scale, algo="split")
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    torch.cuda.synchronize()
    isa.attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, mask=mask, causal=c.causal, softmax_scale=c.scale)
    torch.cuda.synchronize()
    return [dev_to_f64(t) for t in ref], [dev_to_f64(t) for t in (dq, dk, dv)]


def test_noalloc_two_calls_match_split():
    for name, case, exact in CALLS:
        c = build_case(case)
        log(f"noalloc {name} [{c.label()}]")
        ref, got = run_both(c)
        orc = oracle_grads(c)
        for n, g, r, o in zip(("dq", "dk", "dv"), got, ref, orc):
            assert_close(f"{n} vs split", g, r)
            assert_close(f"{n} vs oracle", g, o)
            if exact:
                assert np.array_equal(g, r), f"{name}: {n} differs from the existing entry point"
