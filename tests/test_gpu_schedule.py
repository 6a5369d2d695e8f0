"""GPU parity where the dK/dV work order groups items by head and lets the
longest ones run first: 2048 (batch, KV head, key block) items, i.e. at least
8 per CU of each XCD, and a "sink" key block that every query block keeps, so
its items carry far more than twice the mean work.  The order changes no
arithmetic, so the usual tolerance against the fp64 oracle applies; one
query head carries real forward statistics and is checked element by
element, every other head gets LSE = +inf and must come out exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_close, bits_to_dev, csr_to_host, assert_csr_equal, dev_to_f64, log

pytestmark = pytest.mark.gpu

B, H, S, D = 1, 32, 8192, 64
CHECKED = [5]
_case = {}


def sink_case():
    if _case:
        return _case
    g = synth.seed_streams(41)
    n = S // 128
    pres = (g[4].random((B, H, n, n)) < 0.08).astype(np.uint8)
    pres[..., np.arange(n), np.arange(n)] = 1          # the diagonal
    pres[..., :, 0] = 1                                 # the sink: key block 0 for every query block
    d = {"q": synth.bf16_normal(g[0], (B, S, H, D)), "k": synth.bf16_normal(g[1], (B, S, H, D)),
         "v": synth.bf16_normal(g[2], (B, S, H, D)), "do": synth.bf16_normal(g[3], (B, S, H, D)),
         "presence": pres}
    d["csr"] = oracle.presence_to_csr(pres)
    omask = oracle.block_mask_from_csr(H, *d["csr"])
    scale = float(np.float32(1.0 / np.sqrt(D)))
    f = {k: oracle.bf16_to_f64(d[k]) for k in ("q", "k", "v", "do")}
    log(f"sink mask: oracle forward/backward of heads {CHECKED}")
    O, L = oracle.attn_fwd(f["q"], f["k"], f["v"], omask, False, scale, heads=CHECKED)
    d["o"] = oracle.round_to_bf16(O)
    d["lse"] = oracle.round_to_f32(L)
    d["ref"] = oracle.attn_bwd(f["q"], f["k"], f["v"], oracle.bf16_to_f64(d["o"]), f["do"],
                               d["lse"].astype(np.float64), omask, False, scale, heads=CHECKED)
    d["scale"] = scale
    _case.update(d)
    return _case


@pytest.mark.parametrize("algo", ["split", "split_ds"])
def test_sink_mask_grouped_order(algo):
    import index_sparse_attention_amd as isa
    d = sink_case()
    log(f"sink mask {algo}")
    mask = isa.block_mask_to_csr(torch.from_numpy(d["presence"]).cuda())
    assert_csr_equal(csr_to_host(mask), d["csr"])
    q, k, v = bits_to_dev(d["q"]), bits_to_dev(d["k"]), bits_to_dev(d["v"])
    # outputs and workspace start as NaN: a block no work item writes stays NaN
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    ws = torch.full((isa.attn_bwd_workspace_bytes(B, S, S, H, H, D, D, algo),), 0xFF, dtype=torch.uint8,
                    device=q.device)
    isa.attn_bwd(q, k, v, bits_to_dev(d["o"]), bits_to_dev(d["do"]), torch.from_numpy(d["lse"]).cuda(), mask=mask,
                 causal=False, softmax_scale=d["scale"], algo=algo, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    # the work order: each XCD's slice of each pass is a permutation of its item range
    n_items = B * H * (S // 128)
    stat_bytes = B * H * S * 4                          # delta, then lse * log2(e); 256-byte multiples here
    order = ws[2 * stat_bytes:2 * stat_bytes + 8 * n_items].view(torch.int32).cpu().numpy()
    per = -(-n_items // 8)
    for pass_, base in (("dK/dV", 0), ("dQ", n_items)):
        for x in range(8):
            lo, hi = min(n_items, x * per), min(n_items, (x + 1) * per)
            got = np.sort(order[base + lo:base + hi])
            assert np.array_equal(got, np.arange(lo, hi)), f"{pass_} order of XCD {x} is not a permutation"
    dq, dk, dv = dev_to_f64(dq), dev_to_f64(dk), dev_to_f64(dv)
    rq, rk, rv = d["ref"]
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_close(f"{name}[checked head]", got[:, :, CHECKED], ref[:, :, CHECKED])
    others = [h for h in range(H) if h not in CHECKED]
    assert np.all(dq[:, :, others] == 0) and np.all(dk[:, :, others] == 0) and np.all(dv[:, :, others] == 0)
