"""GPU parity of the index -> block CSR converter and the block-mask -> CSR
compaction: bit-exact against the oracle (integer work)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import assert_csr_equal, csr_to_host, log

pytestmark = pytest.mark.gpu


def _gpu_index(indices, B, Sq, Sk, bq=128, bk=128):
    import index_sparse_attention_amd as isa
    m = isa.index_to_block_sparse(torch.from_numpy(np.ascontiguousarray(indices)).cuda(), B, Sq, Sk, bq, bk)
    torch.cuda.synchronize()
    return csr_to_host(m)


def _oracle_index(indices, B, Sq, Sk, bq=128, bk=128):
    return oracle.presence_to_csr(oracle.indices_to_presence(indices, B, Sq, Sk, bq, bk))


def _structured(kind, B, Sq, Sk, nhk, topk, rng):
    idx = np.full((B * Sq, nhk, topk), -1, dtype=np.int32)
    rows = np.arange(B * Sq) % Sq
    if kind == "local_window":
        for t in range(topk):
            idx[:, :, t] = np.clip(rows - t, -1, None)[:, None]
    elif kind == "strided":
        for t in range(topk):
            idx[:, :, t] = ((rows * 7 + t * 129) % Sk)[:, None]
    elif kind == "all_padding":
        pass
    elif kind == "duplicates":
        idx[:, :, :] = (rows % Sk)[:, None, None]
    elif kind == "out_of_range":
        idx[:] = rng.integers(-5, 2 * Sk, size=idx.shape)
        idx[idx == Sk + 3] = np.iinfo(np.int32).max
        idx[idx == -3] = np.iinfo(np.int32).min
    elif kind == "shuffled_full_causal":
        for r in range(B * Sq):
            i = r % Sq
            valid = np.arange(min(i + 1, topk))
            idx[r, :, :len(valid)] = rng.permutation(valid)[None, :]
    return idx


@pytest.mark.parametrize("kind", ["local_window", "strided", "all_padding", "duplicates", "out_of_range",
                                  "shuffled_full_causal"])
@pytest.mark.parametrize("shape", [(1, 300, 300, 2, 8), (2, 128, 515, 1, 5), (1, 1, 1, 1, 4)])
def test_index_converter_structured(kind, shape):
    B, Sq, Sk, nhk, topk = shape
    rng = np.random.default_rng(11)
    idx = _structured(kind, B, Sq, Sk, nhk, topk, rng)
    log(f"converter structured {kind} {shape}")
    assert_csr_equal(_gpu_index(idx, B, Sq, Sk), _oracle_index(idx, B, Sq, Sk))


@pytest.mark.parametrize("seed", range(4))
def test_index_converter_random(seed):
    rng = np.random.default_rng(seed)
    B, Sq, Sk, nhk = int(rng.integers(1, 3)), int(rng.integers(1, 700)), int(rng.integers(1, 900)), int(rng.integers(1, 4))
    topk = int(rng.integers(1, 70))
    bq, bk = [(128, 128), (64, 32), (7, 13), (128, 1)][seed]
    idx = synth.topk_indices(rng, B, Sq, Sk, nhk, topk, causal=bool(seed % 2))
    log(f"converter random B{B} Sq{Sq} Sk{Sk} nhk{nhk} topk{topk} block{bq}x{bk}")
    assert_csr_equal(_gpu_index(idx, B, Sq, Sk, bq, bk), _oracle_index(idx, B, Sq, Sk, bq, bk))


def test_index_converter_scalar_path_and_zero_topk():
    """topk not a multiple of 4 takes the scalar load path; topk = 0 gives empty lists."""
    rng = np.random.default_rng(5)
    idx = synth.topk_indices(rng, 1, 400, 400, 2, 7)
    assert_csr_equal(_gpu_index(idx, 1, 400, 400), _oracle_index(idx, 1, 400, 400))
    empty = np.zeros((400, 2, 0), dtype=np.int32)
    got = _gpu_index(empty, 1, 400, 400)
    assert_csr_equal(got, _oracle_index(empty, 1, 400, 400))
    assert got[0][-1] == 0


def test_index_converter_repeatable():
    rng = np.random.default_rng(9)
    idx = synth.topk_indices(rng, 1, 1000, 1000, 2, 100)
    a = _gpu_index(idx, 1, 1000, 1000)
    b = _gpu_index(idx, 1, 1000, 1000)
    assert_csr_equal(a, b)


def test_index_converter_full_workload():
    """top-2048 indices over 16K causal tokens, 2 KV heads (256 MiB of int32)."""
    w = synth.WORKLOADS["indexsparse_gqa_s16k_d128"]
    idx = synth.make_workload_inputs(w, want=("mask",))["indices"]
    log(f"converter full workload {idx.shape}")
    got = _gpu_index(idx, w.batch, w.seqlen_q, w.seqlen_k)
    ref = _oracle_index(idx, w.batch, w.seqlen_q, w.seqlen_k)
    assert_csr_equal(got, ref)
    assert int(got[0][-1]) == 2 * 128 * 129 // 2      # the full lower block triangle per KV head


# up to (1, 1, 4, 1024) the shapes fit the single-launch path (slices of at
# most 1024 x 1024 and 4 KiB, 256 KiB in all; (4, 16, 64, 64) at the total
# and the last two at the row and column limits); the rest take the count /
# scan / fill launches
@pytest.mark.parametrize("shape", [(2, 16, 64, 64), (1, 3, 5, 9), (3, 1, 70, 1), (1, 2, 1, 130), (1, 1, 129, 2),
                                   (4, 16, 64, 64), (1, 1, 1024, 4), (1, 1, 4, 1024),
                                   (1, 4, 128, 128), (2, 3, 100, 77), (1, 1, 1024, 16), (1, 1, 16, 1024),
                                   (8, 16, 64, 64), (1, 1, 2000, 3), (1, 1, 3, 2000), (1, 2, 128, 200)])
def test_block_mask_to_csr(shape):
    import index_sparse_attention_amd as isa
    rng = np.random.default_rng(sum(shape))
    pres = (rng.random(shape) < 0.3).astype(np.uint8) * rng.integers(1, 255, size=shape).astype(np.uint8)
    log(f"block mask csr {shape}")
    m = isa.block_mask_to_csr(torch.from_numpy(pres).cuda())
    torch.cuda.synchronize()
    assert_csr_equal(csr_to_host(m), oracle.presence_to_csr(pres))


@pytest.mark.parametrize("offset", [1, 16])
def test_block_mask_to_csr_unaligned(offset):
    """A presence view that starts off a 16-byte boundary takes the byte loads."""
    import index_sparse_attention_amd as isa
    shape = (3, 4, 32, 32)
    rng = np.random.default_rng(offset)
    pres = (rng.random(shape) < 0.4).astype(np.uint8)
    flat = torch.zeros(offset + pres.size, dtype=torch.uint8, device="cuda")
    flat[offset:] = torch.from_numpy(pres.reshape(-1)).cuda()
    view = flat[offset:].view(shape)
    log(f"block mask csr unaligned offset {offset}")
    m = isa.block_mask_to_csr(view)
    torch.cuda.synchronize()
    assert_csr_equal(csr_to_host(m), oracle.presence_to_csr(pres))


def test_index_converter_large_path():
    """More than 1024 key blocks: the index path's count / scan / fill launches
    (with the row counts the presence kernel already produced)."""
    rng = np.random.default_rng(21)
    B, Sq, Sk, nhk, topk = 2, 200, 2100, 2, 9
    idx = synth.topk_indices(rng, B, Sq, Sk, nhk, topk)
    log("converter large path")
    assert_csr_equal(_gpu_index(idx, B, Sq, Sk, 64, 2), _oracle_index(idx, B, Sq, Sk, 64, 2))
