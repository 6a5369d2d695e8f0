"""Seeded synthetic inputs for the attention-backward workloads.

This package only draws random numbers and lays them out: bf16 Gaussian
tensors, Bernoulli block masks and top-k token index lists.  It holds none of
the attention arithmetic, so both the fp64 oracle and the HIP path can consume
its output without sharing any computation.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    bf16_normal,
    block_mask,
    seed_streams,
    topk_indices,
    make_workload_inputs,
)
