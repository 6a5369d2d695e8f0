"""Pins for the oracle's bf16/fp32 edge conversions and the synthetic generators."""
import numpy as np
import torch

import oracle
import synth


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000, 0x4049],
                    dtype=np.uint16)
    got = oracle.bf16_to_f64(bits)
    exp = [1.0, -2.0, np.inf, -np.inf, 2.0 ** -133, 0.0, -0.0, 3.140625]
    np.testing.assert_array_equal(got, exp)


def test_bf16_rounding_ties_and_edges():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2 ** -8: 0x3F80,                  # halfway, tie to even (down)
        one + 3 * 2 ** -8: 0x3F82,              # halfway, tie to even (up)
        one + 2 ** -8 + 2 ** -30: 0x3F81,       # just above halfway
        -(one + 2 ** -7): 0xBF81,
        3.5e38: 0x7F80,                         # beyond the largest bf16 -> inf
        2.0 ** -133: 0x0001,                    # smallest subnormal
        1.5 * 2.0 ** -134: 0x0001,              # between 0 and 2^-133, rounds up
        0.0: 0x0000,
    }
    x = np.array(list(cases.keys()))
    got = oracle.round_to_bf16(x)
    assert got.tolist() == list(cases.values())
    assert oracle.round_to_bf16(np.array([np.nan]))[0] == 0x7FC0


def test_bf16_rounding_vs_torch_and_synth():
    """Three independent roundings agree on float32 inputs: the oracle's
    (float64 grid arithmetic), synth's (integer bit arithmetic) and torch's cast."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    a = oracle.round_to_bf16(x.astype(np.float64))
    b = synth.bf16_bits_from_f32(x)
    c = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
    np.testing.assert_array_equal(oracle.bf16_to_f64(a), torch.from_numpy(x).to(torch.bfloat16)
                                  .to(torch.float64).numpy())


def test_synth_streams_are_seeded():
    w = synth.WORKLOADS["dense_mha_s256_d64"]
    a = synth.make_workload_inputs(w)
    b = synth.make_workload_inputs(w)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (1, 256, 2, 64) and a["q"].dtype == np.uint16


def test_synth_topk_indices_are_uniform_causal_samples():
    rng = np.random.default_rng(3)
    Sq = Sk = 300
    idx = synth.topk_indices(rng, 1, Sq, Sk, 2, 64)
    assert idx.shape == (300, 2, 64) and idx.dtype == np.int32
    for i in range(Sq):
        for h in range(2):
            row = idx[i, h]
            valid = row[row >= 0]
            assert len(valid) == min(64, i + 1)
            assert len(set(valid.tolist())) == len(valid)
            assert valid.max() <= i
            assert np.all(row[len(valid):] == -1)
    # order of the selected positions is not positional
    assert not all(np.all(np.diff(idx[i, 0]) > 0) for i in range(100, 300))


def test_synth_block_mask():
    rng = np.random.default_rng(4)
    m = synth.block_mask(rng, 2, 3, 64, 64, 0.25, True)
    assert m.dtype == np.uint8 and m.shape == (2, 3, 64, 64)
    assert np.all(m[:, :, np.arange(64), np.arange(64)] == 1)
    frac = (m.sum() - 2 * 3 * 64) / (2 * 3 * 64 * 63)
    assert 0.22 < frac < 0.28
