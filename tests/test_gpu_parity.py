"""GPU parity of the attention backward against the fp64 oracle, at sizes the
oracle finishes in seconds (several 128-row tiles plus ragged tails), for
dense / causal / GQA / block-sparse / index-sparse masks and both loop orders."""
import numpy as np
import pytest

from tests.gpu_helpers import (Case, assert_close, assert_csr_equal, build_case, csr_to_host, gpu_mask,
                               log, oracle_grads, run_gpu)

pytestmark = pytest.mark.gpu

CASES = {
    "dense_mha_s256_d64": Case(1, 256, 256, 2, 2, 64, 64, seed=1),
    "dense_ragged_d128": Case(1, 300, 300, 2, 2, 128, 128, seed=2),
    "dense_b2_d128": Case(2, 256, 200, 2, 1, 128, 128, seed=3),
    "causal_gqa_br_d128": Case(1, 200, 333, 4, 2, 128, 128, causal=True, seed=4),
    "causal_sq_gt_sk_d64": Case(1, 333, 200, 2, 1, 64, 64, causal=True, seed=5),
    "causal_square_d128": Case(2, 384, 384, 2, 2, 128, 128, causal=True, seed=6),
    "block_hq_ragged_d128": Case(1, 520, 520, 2, 2, 128, 128, mask="block", keep=0.4, seed=7),
    "block_h1_gqa_causal": Case(1, 512, 512, 4, 2, 128, 128, causal=True, mask="block", Hm=1, keep=0.5, seed=8),
    "block_hk_gqa_d64": Case(2, 256, 384, 4, 2, 64, 64, mask="block", Hm=2, keep=0.5, seed=9),
    "index_gqa_d128": Case(1, 640, 640, 4, 2, 128, 128, mask="index", topk=96, seed=10),
    "index_gqa_causal_d128": Case(1, 512, 512, 4, 1, 128, 128, causal=True, mask="index", topk=48, seed=11),
    "causal_d192": Case(1, 384, 384, 2, 2, 192, 128, causal=True, seed=12),
    "dense_ragged_d192": Case(1, 200, 330, 2, 1, 192, 128, seed=13),
    "block_d192": Case(1, 512, 512, 2, 2, 192, 128, mask="block", keep=0.5, seed=14),
    "tiny_1x1": Case(1, 1, 1, 1, 1, 64, 64, seed=15),
    "sk_one": Case(1, 130, 1, 2, 2, 128, 128, seed=16),
    "sq_one_causal": Case(1, 1, 257, 2, 2, 128, 128, causal=True, seed=17),
    # 512 or more (b, KV head, key block) items: the SPLIT dK/dV pass runs one
    # workgroup per item in the per-XCD order; the cases above (fewer items)
    # cut items into parts with fp32 partials and a reduction
    "many_items_dense": Case(4, 256, 256, 64, 64, 128, 128, seed=18),
    "many_items_causal_ragged": Case(4, 256, 320, 64, 64, 128, 128, causal=True, seed=19),
    "many_items_block_gqa": Case(2, 256, 256, 256, 128, 64, 64, mask="block", Hm=128, keep=0.5, seed=20),
}

_built = {}


def get_case(name):
    if name not in _built:
        _built[name] = build_case(CASES[name])
    return _built[name]


@pytest.mark.parametrize("algo", ["loopk", "loopq", "split", "split_ds"])
@pytest.mark.parametrize("name", list(CASES))
def test_attn_bwd_parity(name, algo):
    c = get_case(name)
    log(f"parity {name} [{c.label()}] algo={algo}")
    mask = gpu_mask(c)
    if mask is not None:
        assert_csr_equal(csr_to_host(mask), c.data["csr"])
    dq, dk, dv = run_gpu(c, algo, mask)
    rq, rk, rv = oracle_grads(c)
    assert_close("dq", dq, rq)
    assert_close("dk", dk, rk)
    assert_close("dv", dv, rv)


@pytest.mark.parametrize("name", ["causal_gqa_br_d128", "block_h1_gqa_causal", "index_gqa_d128", "causal_d192"])
def test_loop_orders_agree(name):
    """LoopK, LoopQ and both split variants agree within the tolerance (fp32
    accumulation order differs between them)."""
    c = get_case(name)
    log(f"loopk vs loopq vs split {name}")
    mask = gpu_mask(c)
    a = run_gpu(c, "loopk", mask)
    for other in ("loopq", "split", "split_ds"):
        b = run_gpu(c, other, mask)
        for n, x, y in zip(("dq", "dk", "dv"), a, b):
            assert_close(f"{n} loopk-vs-{other}", x, y)


@pytest.mark.parametrize("algo", ["loopk", "loopq", "split", "split_ds"])
def test_dense_equals_all_kept_blocks(algo):
    """Dense mask and an all-kept block mask give the same gradients."""
    import torch
    import index_sparse_attention_amd as isa
    c = get_case("dense_ragged_d128")
    pres = np.ones((c.B, c.Hq, 3, 3), dtype=np.uint8)
    m = isa.block_mask_to_csr(torch.from_numpy(pres).cuda())
    a = run_gpu(c, algo, None)
    b = run_gpu(c, algo, m)
    for n, x, y in zip(("dq", "dk", "dv"), a, b):
        assert_close(n + " dense-vs-allkept", x, y)


@pytest.mark.parametrize("algo", ["loopk", "loopq", "split", "split_ds"])
def test_poisoned_workspace(algo):
    """A workspace full of NaN bytes on entry does not leak into the results."""
    c = get_case("causal_gqa_br_d128")
    log(f"poisoned workspace {algo}")
    dq, dk, dv = run_gpu(c, algo, None, workspace_fill=0xFF)
    rq, rk, rv = oracle_grads(c)
    assert_close("dq", dq, rq)
    assert_close("dk", dk, rk)
    assert_close("dv", dv, rv)


@pytest.mark.parametrize("name", ["block_h1_gqa_causal", "index_gqa_d128", "block_d192"])
def test_split_ds_poisoned_workspace_sparse(name):
    """SPLIT_DS reads back only the dS tiles its dK/dV pass wrote: with a
    NaN-filled workspace the tiles of dropped blocks must never be read."""
    c = get_case(name)
    log(f"poisoned workspace split_ds {name}")
    dq, dk, dv = run_gpu(c, "split_ds", gpu_mask(c), workspace_fill=0xFF)
    rq, rk, rv = oracle_grads(c)
    assert_close("dq", dq, rq)
    assert_close("dk", dk, rk)
    assert_close("dv", dv, rv)


@pytest.mark.parametrize("algo", ["loopk", "loopq", "split", "split_ds"])
def test_empty_sequences(algo):
    """Sq = 0 gives zero dK/dV; Sk = 0 gives zero dQ; B = 0 is a no-op."""
    import torch
    import index_sparse_attention_amd as isa
    bf = dict(dtype=torch.bfloat16, device="cuda")
    for Sq, Sk in ((0, 130), (130, 0)):
        q = torch.randn(1, Sq, 2, 64, **bf)
        k = torch.randn(1, Sk, 2, 64, **bf)
        v = torch.randn(1, Sk, 2, 64, **bf)
        o = torch.randn(1, Sq, 2, 64, **bf)
        lse = torch.full((1, 2, Sq), float("inf"), dtype=torch.float32, device="cuda")
        dq = torch.full_like(q, 7.0)
        dk = torch.full_like(k, 7.0)
        dv = torch.full_like(v, 7.0)
        isa.attn_bwd(q, k, v, o, o, lse, algo=algo, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)
    q = torch.randn(0, 16, 2, 64, **bf)
    isa.attn_bwd(q, q, q, q, q, torch.zeros(0, 2, 16, device="cuda"), algo=algo)


@pytest.mark.parametrize("algo", ["split", "split_ds"])
@pytest.mark.parametrize("name", ["block_h1_gqa_causal", "index_gqa_d128", "many_items_block_gqa", "causal_d192"])
def test_split_is_bit_reproducible(name, algo):
    """The atomic-free algorithms are deterministic: every reduction (dQ over
    key blocks, dK/dV over query blocks and heads, part-mode partials) runs in
    a fixed order, so repeated calls -- also with a NaN-filled workspace --
    give bit-identical dQ, dK and dV.  (LoopK/LoopQ reduce with fp32 atomics
    and are only reproducible up to rounding.)"""
    c = get_case(name)
    log(f"bit reproducibility {algo} {name}")
    mask = gpu_mask(c)
    first = run_gpu(c, algo, mask)
    for fill in (None, 0xFF, None):
        again = run_gpu(c, algo, mask, workspace_fill=fill)
        for n, x, y in zip(("dq", "dk", "dv"), first, again):
            assert np.array_equal(x, y), f"{algo} {name}: {n} differs between calls"


def test_split_ds_undercounted_blocks_write_nothing():
    """A block CSR whose host-side block count is below the true one (the
    workspace then holds too few dS tiles): the position-map kernel flags it
    and both SPLIT_DS passes compute nothing, so the outputs keep what they
    held and nothing lands past the workspace; the same call with the true
    count is exact again.  (The condition is set from the host; every kernel
    exits normally.)"""
    import torch
    import index_sparse_attention_amd as isa
    from tests.gpu_helpers import bits_to_dev, dev_to_f64
    c = get_case("block_h1_gqa_causal")
    d = c.data
    mask = gpu_mask(c)
    true_nnz = mask.nnz()
    q, k, v = bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"])
    o, do = bits_to_dev(d["o"]), bits_to_dev(d["do"])
    lse = torch.from_numpy(np.ascontiguousarray(d["lse"])).cuda()
    mask.nnz_host = true_nnz - 1
    need = isa.attn_bwd_workspace_bytes(c.B, c.Sq, c.Sk, c.Hq, c.Hk, c.Dqk, c.Dv, "split_ds", mask=mask,
                                        causal=c.causal)
    # a guard region after the workspace: must stay untouched
    buf = torch.full((need + (1 << 20),), 0x5A, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.full_like(t, 3.0) for t in (q, k, v))
    isa.attn_bwd(q, k, v, o, do, lse, mask=mask, causal=c.causal, softmax_scale=c.scale, algo="split_ds",
                 dq=dq, dk=dk, dv=dv, workspace=buf[:need])
    torch.cuda.synchronize()
    assert torch.all(dq == 3.0) and torch.all(dk == 3.0) and torch.all(dv == 3.0)
    assert torch.all(buf[need:] == 0x5A), "a write landed past the workspace"
    mask.nnz_host = true_nnz
    got = run_gpu(c, "split_ds", mask, workspace_fill=0xFF)
    for n, g, r in zip(("dq", "dk", "dv"), got, oracle_grads(c)):
        assert_close(n, g, r)
