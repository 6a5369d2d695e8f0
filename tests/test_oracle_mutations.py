"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check
that the pins in test_oracle_attention.py / test_oracle_convert.py detect them.

A pin set that still passes with a planted mistake would not pin anything; each
case below must make at least one pin fail.
"""
import json
import os

import numpy as np
import pytest

import oracle
import oracle.attention as oa
import oracle.convert as oc
import oracle.masks as om
from tests.test_oracle_attention import _fd_check, block_spec


def _golden_attn_ok(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)
    arr = lambda key: np.asarray(g[key], dtype=np.float64)
    if "presence" in g:
        mask = oracle.block_mask_from_csr(g["mask_heads"], g["q2k_row_ptr"], g["q2k_col"],
                                          g["k2q_row_ptr"], g["k2q_col"], g["block"], g["block"])
    else:
        mask = oracle.dense_mask()
    O, L = oracle.attn_fwd(arr("q"), arr("k"), arr("v"), mask, g["causal"], g["scale"])
    grads = oracle.attn_bwd(arr("q"), arr("k"), arr("v"), O, arr("do"), L, mask, g["causal"],
                            g["scale"])
    e = g["expected"]
    ok = np.allclose(O, e["o"], atol=1e-12) and np.allclose(L, e["lse"], atol=1e-12)
    for got, key in zip(grads, ("dq", "dk", "dv")):
        ok = ok and np.allclose(got, e[key], atol=1e-12)
    return ok


def _all_golden_ok(golden_dir):
    names = ["attn_two_keys.json", "attn_causal_bottom_right.json",
             "attn_gqa_head_map.json", "attn_block_sparse.json"]
    return all(_golden_attn_ok(golden_dir, n) for n in names)


def _fd_ok(kind="block_Hq"):
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal(s) for s in [(1, 5, 2, 3), (1, 7, 1, 3), (1, 7, 1, 2),
                                                    (1, 5, 2, 2)])
    if kind == "dense_causal":
        mask, causal = oracle.dense_mask(), True
    else:
        pres = (rng.random((1, 2, 3, 4)) < 0.6).astype(np.uint8)
        pres[..., 0] = 1
        mask, causal = block_spec(pres, 2, 2), False
    try:
        _fd_check(q, k, v, do, mask, causal, 0.61)
        return True
    except AssertionError:
        return False


def test_unmutated_oracle_passes(golden_dir):
    assert _all_golden_ok(golden_dir) and _fd_ok() and _fd_ok("dense_causal")


def test_mutation_ds_sign(monkeypatch, golden_dir):
    orig = oa.tile_grads

    def bad(*a):
        P, dS = orig(*a)
        return P, -dS
    monkeypatch.setattr(oa, "tile_grads", bad)
    assert not (_all_golden_ok(golden_dir) and _fd_ok())


def test_mutation_dropped_delta(monkeypatch, golden_dir):
    orig = oa.tile_grads

    def bad(qr, dor, lser, dr, kc, vc, em, s):
        return orig(qr, dor, lser, np.zeros_like(dr), kc, vc, em, s)
    monkeypatch.setattr(oa, "tile_grads", bad)
    assert not (_all_golden_ok(golden_dir) and _fd_ok())


def test_mutation_scale_outside_exponent(monkeypatch, golden_dir):
    orig = oa.tile_grads

    def bad(qr, dor, lser, dr, kc, vc, em, s):
        return orig(qr, dor, lser, dr, kc, vc, em, 1.0)
    monkeypatch.setattr(oa, "tile_grads", bad)
    assert not (_all_golden_ok(golden_dir) and _fd_ok())


def test_mutation_top_left_causal(monkeypatch, golden_dir):
    def bad(rows, cols, seqlen_q, seqlen_k, causal):
        r = np.asarray(rows)[:, None]
        c = np.asarray(cols)[None, :]
        m = (r < seqlen_q) & (c < seqlen_k)
        if causal:
            m &= c <= r
        return m
    monkeypatch.setattr(om, "element_mask", bad)
    assert not _all_golden_ok(golden_dir)


def test_mutation_interleaved_gqa(monkeypatch, golden_dir):
    monkeypatch.setattr(om, "kv_head", lambda h, hq, hk: h % hk)
    assert not _all_golden_ok(golden_dir)


def test_mutation_transposed_presence(monkeypatch, golden_dir):
    def bad(mask, b, hm, qb, n_qb, n_kb):
        if mask.kind == "dense":
            return np.arange(n_kb)
        r = (b * mask.heads + hm) * n_kb + qb
        return mask.k2q_col[mask.k2q_row_ptr[r]:mask.k2q_row_ptr[r + 1]]
    monkeypatch.setattr(om, "q2k_row", bad)
    assert not _all_golden_ok(golden_dir)


def test_mutation_block_index_off_by_one(monkeypatch, golden_dir):
    """Converter: kb = (idx + 1) // block_k instead of idx // block_k."""
    orig = oc.indices_to_presence

    def bad(indices, batch, seqlen_q, seqlen_k, block_q=128, block_k=128):
        idx = np.asarray(indices).copy()
        valid = (idx >= 0) & (idx < seqlen_k)
        idx[valid] = np.minimum(idx[valid] + 1, seqlen_k - 1)
        return orig(idx, batch, seqlen_q, seqlen_k, block_q, block_k)
    monkeypatch.setattr(oracle, "indices_to_presence", bad)
    with open(os.path.join(golden_dir, "convert_small.json")) as f:
        cases = json.load(f)["cases"]
    ok = True
    for c in cases:
        p = oracle.indices_to_presence(np.asarray(c["indices"]), c["batch"], c["seqlen_q"],
                                       c["seqlen_k"], c["block_q"], c["block_k"])
        ok = ok and p.tolist() == c["presence"]
    assert not ok
