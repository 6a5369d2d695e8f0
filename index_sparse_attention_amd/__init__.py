"""isattn: sparse attention backward for AMD Instinct MI355X (gfx950).

Entry points (thin wrappers over the C ABI in include/isattn.h):

* ``attn_fwd``              -- O and LSE of masked attention (same masks).
* ``attn_bwd``              -- dQ, dK, dV of masked attention (dense, causal,
                               GQA, 128x128 block-sparse); SPLIT_DS, SPLIT,
                               LoopK or LoopQ (``choose_algo`` picks SPLIT_DS
                               when its dS store fits the free memory).
* ``index_to_block_sparse`` -- int32 top-k token indices -> BlockMask (CSR).
* ``block_mask_to_csr``     -- uint8 block presence -> BlockMask (CSR).
* ``topk_select``           -- fp32 score rows -> int32 top-k positions.
"""
from ._abi import LibraryMissing, IsattnError, load as load_library  # noqa: F401
from .api import (  # noqa: F401
    BlockMask,
    Timer,
    attn_bwd,
    attn_bwd_noalloc,
    attn_fwd,
    attn_bwd_workspace_bytes,
    choose_algo,
    block_mask_to_csr,
    index_to_block_sparse,
    topk_select,
)

__version__ = "0.2.0"
