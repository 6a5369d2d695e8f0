"""ctypes declarations of libisattn.so (mirrors include/isattn.h)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libisattn.so")

STATUS = {
    0: "ISATTN_OK", 1: "ISATTN_ERR_NULL", 2: "ISATTN_ERR_SHAPE", 3: "ISATTN_ERR_STRIDE_ALIGN",
    4: "ISATTN_ERR_UNSUPPORTED", 5: "ISATTN_ERR_MASK", 6: "ISATTN_ERR_WORKSPACE",
    7: "ISATTN_ERR_CAPACITY", 8: "ISATTN_ERR_HIP", 9: "ISATTN_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20
MASK_DENSE, MASK_BLOCK_CSR = 0, 1
ALGO_LOOPK, ALGO_LOOPQ, ALGO_SPLIT, ALGO_SPLIT_DS = 0, 1, 2, 3


class Shape(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("seqlen_q", c_int32), ("seqlen_k", c_int32),
                ("heads_q", c_int32), ("heads_k", c_int32), ("dim_qk", c_int32), ("dim_v", c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", c_void_p), ("stride_b", c_int64), ("stride_s", c_int64), ("stride_h", c_int64)]


class Mask(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("block_q", c_int32), ("block_k", c_int32), ("heads", c_int32),
                ("q2k_row_ptr", c_void_p), ("q2k_col", c_void_p),
                ("k2q_row_ptr", c_void_p), ("k2q_col", c_void_p), ("token_bits", c_void_p),
                ("nnz", c_int64)]

    def __init__(self, *args, **kw):
        if len(args) < len(self._fields_) and "nnz" not in kw:
            kw["nnz"] = -1                         # block count unknown unless given
        super().__init__(*args, **kw)


class Varlen(ctypes.Structure):
    _fields_ = [("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p)]


_T = POINTER(Tensor)
_BWD_ARGS = [POINTER(Shape), _T, _T, _T, _T, _T, c_void_p, POINTER(Mask), c_int32, c_float,
             _T, _T, _T, c_int32, c_void_p, c_size_t, c_void_p]

# name -> (restype, argtypes); every function declared in include/isattn.h
SIGNATURES = {
    "isattn_attn_bwd_workspace_bytes": (c_size_t, [POINTER(Shape), c_int32]),
    "isattn_attn_bwd_workspace_bytes_mask": (c_size_t, [POINTER(Shape), c_int32, POINTER(Mask), c_int32, c_int32]),
    "isattn_attn_bwd": (c_int32, _BWD_ARGS),
    "isattn_attn_bwd_timed": (c_int32, _BWD_ARGS + [c_void_p]),
    "isattn_attn_bwd_noalloc": (c_int32, _BWD_ARGS[:13] + [c_void_p]),
    "isattn_attn_fwd": (c_int32, [POINTER(Shape), _T, _T, _T, POINTER(Mask), c_int32, c_float, _T, c_void_p,
                                  c_void_p]),
    "isattn_attn_bwd_varlen": (c_int32, [POINTER(Shape), POINTER(Varlen)] + _BWD_ARGS[1:]),
    "isattn_attn_fwd_varlen": (c_int32, [POINTER(Shape), POINTER(Varlen), _T, _T, _T, POINTER(Mask), c_int32,
                                         c_float, _T, c_void_p, c_void_p]),
    "isattn_index_to_block_sparse_varlen": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                                      c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                                      c_void_p, c_void_p, c_int64, c_void_p, c_size_t,
                                                      c_void_p]),
    "isattn_index_to_block_sparse_workspace_bytes": (c_size_t, [c_int32] * 6),
    "isattn_index_to_block_sparse": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                               c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_int64, c_void_p, c_size_t, c_void_p]),
    "isattn_topk_select": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                                     c_void_p]),
    "isattn_index_to_token_bits": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                             c_void_p, c_void_p, c_int64, c_void_p]),
    "isattn_block_mask_to_csr_workspace_bytes": (c_size_t, [c_int32] * 4),
    "isattn_block_mask_to_csr": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_int64, c_void_p,
                                           c_size_t, c_void_p]),
    "isattn_status_string": (c_char_p, [c_int32]),
    "isattn_version": (c_char_p, []),
    "isattn_timer_create": (c_int32, [c_int32, POINTER(c_void_p)]),
    "isattn_timer_destroy": (c_int32, [c_void_p]),
    "isattn_timer_reset": (c_int32, [c_void_p]),
    "isattn_timer_read": (c_int32, [c_void_p, POINTER(c_int32), POINTER(c_float)]),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load(path: str | None = None):
    """Load libisattn.so (once).  Raises LibraryMissing if it was never built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LibraryMissing(f"{p} is missing: build it with `python -m index_sparse_attention_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class IsattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        lib = load()
        msg = lib.isattn_status_string(code).decode()
        super().__init__(f"{where}: {STATUS.get(code, code)} ({msg})")


def check(code: int, where: str):
    if code != 0:
        raise IsattnError(code, where)
