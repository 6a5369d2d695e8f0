"""fp64 CPU oracle for the masked attention backward and the index->block converter.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library's compute path never
does, and this package imports nothing from the library.

What is computed (the plain definitions, evaluated in float64 with NumPy):

* ``attn_fwd``        -- masked softmax attention: O and the natural-log LSE.
* ``attn_bwd``        -- dQ, dK, dV of that attention given O and LSE, in either
                         of the two loop orders the pages describe ("K order":
                         outer Q blocks, inner kept K blocks; "Q order": outer K
                         blocks, inner kept Q blocks of every head in the group).
* ``indices_to_presence`` / ``presence_to_csr`` -- token top-k indices to a
                         block presence matrix, then to Q->K and K->Q CSR lists.
* ``indices_to_token_mask`` -- the token-exact term: which keys each query's
                         index row selects.
* ``topk_select``     -- the top-k positions of score rows within their
                         [start, end) ranges (the index producer).

Every function names the passage of the source pages it follows.  Readings
where the pages are silent are listed in the module docstrings.
"""
from .numeric import bf16_to_f64, round_to_bf16, round_to_f32  # noqa: F401
from .masks import MaskSpec, dense_mask, block_mask_from_csr, element_mask  # noqa: F401
from .attention import attn_fwd, attn_bwd, flop_count, kept_block_count  # noqa: F401
from .convert import indices_to_presence, indices_to_token_mask, presence_to_csr  # noqa: F401
from .topk import topk_select  # noqa: F401
