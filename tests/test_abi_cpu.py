"""C ABI checks that need no GPU: the library loads, exports every function
include/isattn.h declares, sizes workspaces as documented, and rejects bad
arguments with the documented status before any kernel launch."""
import ctypes
import os
import re

import pytest

from index_sparse_attention_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isattn.h")

OK, NULL, SHAPE, STRIDE, UNSUP, MASK, WS, CAP, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7, 9
FAKE = 0x7F0000000000          # aligned dummy device address: never dereferenced on a failed check


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isattn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), n
        assert n in _abi.SIGNATURES, f"{n} missing from the Python declarations"
    assert set(_abi.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.isattn_version().decode().count(".") == 2
    for code in range(10):
        assert lib.isattn_status_string(code) != b"unknown status"
    assert lib.isattn_status_string(99) == b"unknown status"


def shape(B=1, Sq=256, Sk=256, Hq=2, Hk=2, Dqk=128, Dv=128):
    return _abi.Shape(B, Sq, Sk, Hq, Hk, Dqk, Dv)


def ws_bytes(lib, s, algo):
    return lib.isattn_attn_bwd_workspace_bytes(ctypes.byref(s), algo)


def test_workspace_sizes(lib):
    s = shape(B=2, Sq=300, Sk=200, Hq=4, Hk=2, Dqk=128, Dv=128)
    al = lambda x: (x + 255) // 256 * 256
    delta = al(2 * 300 * 4 * 4)
    assert ws_bytes(lib, s, 0) == delta + al(2 * 200 * 2 * 128 * 4) * 2
    assert ws_bytes(lib, s, 1) == delta + al(2 * 300 * 4 * 128 * 4)
    # SPLIT: delta and lse*log2(e), each padded per (batch, head) to whole 128-row blocks, then the
    # work order of the two passes (B*Hk*n_kb + B*Hq*n_qb int32); with fewer than 512 dK/dV items the
    # part mode adds units, per-item info and fp32 partial slots: items 8, dense query blocks per item
    # G*n_qb = 6, target part T = ceil(sqrt(16 * 6*8 / 256)) = 2, at most 3 parts per item -> 24 slots
    # of 128 x 256
    stats = al(2 * 4 * 384 * 4)
    part_mode = al((24 + 1) * 4) + al(3 * 8 * 4) + al(24 * 128 * (128 + 128) * 4)
    assert ws_bytes(lib, s, 2) == 2 * stats + al((2 * 2 * 2 + 2 * 4 * 3) * 4) + part_mode
    # 512 or more dK/dV items: no part mode
    big = shape(B=1, Sq=128, Sk=128 * 256, Hq=2, Hk=2)
    assert ws_bytes(lib, big, 2) == 2 * al(2 * 128 * 4) + al((2 * 256 + 2 * 1) * 4)
    # SPLIT_DS sized for any mask: SPLIT's parts, an int32 position map and a 128 x 128 bf16 dS tile
    # per (b, h, query block, key block)
    assert ws_bytes(lib, s, 3) == ws_bytes(lib, s, 2) + al(2 * 4 * 3 * 2 * 4 + 4) + al(2 * 4 * 3 * 2 * 128 * 128 * 2)
    assert ws_bytes(lib, big, 3) == ws_bytes(lib, big, 2) + al(2 * 256 * 4 + 4) + al(1 * 2 * 1 * 256 * 128 * 128 * 2)
    assert ws_bytes(lib, s, 7) == 0
    assert lib.isattn_attn_bwd_workspace_bytes(None, 0) == 0
    # converter: presence B*H*nQB*nKB bytes + row and column counts
    assert lib.isattn_index_to_block_sparse_workspace_bytes(1, 16384, 16384, 2, 128, 128) == \
        al(2 * 128 * 128) + al(2 * 128 * 4) + al(2 * 128 * 4)
    assert lib.isattn_block_mask_to_csr_workspace_bytes(2, 16, 64, 64) == al(2 * 16 * 64 * 4) * 2


class Call:
    """Builds a valid-looking isattn_attn_bwd argument set; tests break one part."""

    def __init__(self, lib, algo=0, **kw):
        self.lib = lib
        self.shape = shape(**kw)
        s = self.shape
        self.views = {}
        for name, (S, H, D) in {"q": (s.seqlen_q, s.heads_q, s.dim_qk), "k": (s.seqlen_k, s.heads_k, s.dim_qk),
                                "v": (s.seqlen_k, s.heads_k, s.dim_v), "o": (s.seqlen_q, s.heads_q, s.dim_v),
                                "do": (s.seqlen_q, s.heads_q, s.dim_v), "dq": (s.seqlen_q, s.heads_q, s.dim_qk),
                                "dk": (s.seqlen_k, s.heads_k, s.dim_qk), "dv": (s.seqlen_k, s.heads_k, s.dim_v)}.items():
            self.views[name] = _abi.Tensor(FAKE, S * H * D, H * D, D)
        self.lse = FAKE
        self.mask = None
        self.causal = 0
        self.scale = 0.125
        self.algo = algo
        self.ws = FAKE
        self.ws_bytes = ws_bytes(lib, self.shape, algo) if algo in (0, 1, 2, 3) else 0

    def __call__(self, shape_ptr=True):
        v = self.views
        sp = ctypes.byref(self.shape) if shape_ptr else None
        mp = ctypes.byref(self.mask) if self.mask is not None else None
        ref = lambda t: ctypes.byref(t) if t is not None else None
        return self.lib.isattn_attn_bwd(sp, ref(v["q"]), ref(v["k"]), ref(v["v"]), ref(v["o"]), ref(v["do"]),
                                        self.lse, mp, self.causal, self.scale, ref(v["dq"]), ref(v["dk"]),
                                        ref(v["dv"]), self.algo, self.ws, self.ws_bytes, None)


def test_bwd_validation_errors(lib):
    assert Call(lib)(shape_ptr=False) == NULL
    c = Call(lib); c.views["q"] = None; assert c() == NULL
    c = Call(lib); c.views["dk"].ptr = None; assert c() == NULL
    c = Call(lib); c.lse = None; assert c() == NULL
    assert Call(lib, Hq=3, Hk=2)() == SHAPE
    assert Call(lib, B=-1)() == SHAPE
    assert Call(lib, Dqk=96, Dv=96)() == UNSUP
    assert Call(lib, Dqk=128, Dv=64)() == UNSUP
    assert Call(lib, Dqk=256, Dv=256)() == UNSUP
    assert Call(lib, algo=5)() == UNSUP
    c = Call(lib); c.scale = float("nan"); assert c() == UNSUP
    c = Call(lib); c.views["v"].ptr = FAKE + 8; assert c() == STRIDE
    c = Call(lib); c.views["o"].stride_s = 130; assert c() == STRIDE
    c = Call(lib); c.views["dq"].stride_h = -128; assert c() == STRIDE
    c = Call(lib); c.ws_bytes -= 1; assert c() == WS
    c = Call(lib); c.ws = None; assert c() == WS
    c = Call(lib); c.ws = FAKE + 16; assert c() == WS
    c = Call(lib); c.mask = _abi.Mask(7, 128, 128, 2, FAKE, FAKE, FAKE, FAKE); assert c() == MASK
    c = Call(lib); c.mask = _abi.Mask(1, 64, 64, 2, FAKE, FAKE, FAKE, FAKE); assert c() == UNSUP
    c = Call(lib, Hq=4, Hk=2); c.mask = _abi.Mask(1, 128, 128, 3, FAKE, FAKE, FAKE, FAKE); assert c() == MASK
    c = Call(lib); c.mask = _abi.Mask(1, 128, 128, 2, None, None, FAKE, FAKE); assert c() == NULL
    c = Call(lib, algo=1); c.mask = _abi.Mask(1, 128, 128, 2, FAKE, FAKE, None, None); assert c() == NULL
    # SPLIT addresses a head's Q/dO/K/V rows with 32-bit byte offsets: (rows rounded up to 128) x stride x 2
    # must stay below 2^31 (here 256 rows x 2^22 x 2 = 2^31)
    c = Call(lib, algo=2); c.views["q"].stride_s = 1 << 22; c.views["q"].stride_b = 256 << 22
    assert c() == STRIDE
    c = Call(lib, algo=2); c.views["do"].stride_s = 1 << 22; c.views["do"].stride_b = 256 << 22
    assert c() == STRIDE
    c = Call(lib, algo=2); c.views["k"].stride_s = 1 << 22; c.views["k"].stride_b = 256 << 22
    assert c() == STRIDE
    c = Call(lib, algo=2); c.views["v"].stride_s = 1 << 22; c.views["v"].stride_b = 256 << 22
    assert c() == STRIDE
    c = Call(lib, algo=2); c.ws_bytes -= 1; assert c() == WS
    c = Call(lib, algo=3); c.views["k"].stride_s = 1 << 22; c.views["k"].stride_b = 256 << 22
    assert c() == STRIDE
    c = Call(lib, algo=3); c.ws_bytes = ws_bytes(lib, shape(), 2) - 1; assert c() == WS
    c = Call(lib, algo=3); c.mask = _abi.Mask(1, 128, 128, 2, FAKE, FAKE, None, None); assert c() == NULL


def test_fwd_validation_errors(lib):
    s = shape()
    views = {n: _abi.Tensor(FAKE, 256 * 2 * 128, 2 * 128, 128) for n in ("q", "k", "v", "o")}

    def call(shape_ptr=True, lse=FAKE, mask=None, scale=0.125, **over):
        vv = dict(views, **over)
        ref = lambda t: ctypes.byref(t) if t is not None else None
        return lib.isattn_attn_fwd(ctypes.byref(s) if shape_ptr else None, ref(vv["q"]), ref(vv["k"]),
                                   ref(vv["v"]), ctypes.byref(mask) if mask is not None else None, 0, scale,
                                   ref(vv["o"]), lse, None)
    assert call(shape_ptr=False) == NULL
    assert call(q=None) == NULL
    assert call(lse=None) == NULL
    assert call(o=_abi.Tensor(FAKE + 8, 0, 256, 128)) == STRIDE
    assert call(scale=float("inf")) == UNSUP
    assert call(mask=_abi.Mask(7, 128, 128, 2, FAKE, FAKE, None, None)) == MASK
    assert call(mask=_abi.Mask(1, 128, 128, 2, None, None, FAKE, FAKE)) == NULL
    assert call(mask=_abi.Mask(1, 64, 64, 2, FAKE, FAKE, None, None)) == UNSUP
    assert call(k=_abi.Tensor(FAKE, 0, 1 << 22, 128)) == STRIDE     # 256 rows x 2^22 x 2 B = 2^31


def test_index_converter_validation_errors(lib):
    def call(indices=FAKE, B=1, Sq=256, Sk=256, nhk=2, topk=64, bq=128, bk=128, cap=None, ws=FAKE,
             wsb=None, outs=(FAKE, FAKE, FAKE, FAKE)):
        n_qb, n_kb = -(-Sq // max(bq, 1)), -(-Sk // max(bk, 1))
        cap = B * nhk * n_qb * n_kb if cap is None else cap
        if wsb is None:
            wsb = lib.isattn_index_to_block_sparse_workspace_bytes(B, Sq, Sk, nhk, max(bq, 1), max(bk, 1))
        return lib.isattn_index_to_block_sparse(indices, B, Sq, Sk, nhk, topk, bq, bk, *outs, cap, ws, wsb,
                                                None)
    assert call(indices=None) == NULL
    assert call(outs=(None, FAKE, FAKE, FAKE)) == NULL
    assert call(outs=(FAKE, FAKE, FAKE, None)) == NULL
    assert call(B=-1) == SHAPE
    assert call(bq=0) == SHAPE
    assert call(cap=7) == CAP
    assert call(wsb=16) == WS
    assert call(ws=FAKE + 64) == WS
    assert call(Sk=(1 << 19) * 128 + 1, bk=128) == UNSUP


def test_block_mask_validation_errors(lib):
    def call(presence=FAKE, B=2, H=4, nq=8, nk=8, cap=None, wsb=None, ws=FAKE):
        cap = B * H * nq * nk if cap is None else cap
        wsb = lib.isattn_block_mask_to_csr_workspace_bytes(B, H, nq, nk) if wsb is None else wsb
        return lib.isattn_block_mask_to_csr(presence, B, H, nq, nk, FAKE, FAKE, FAKE, FAKE, cap, ws, wsb, None)
    assert call(presence=None) == NULL
    assert call(H=-2) == SHAPE
    assert call(cap=10) == CAP
    assert call(wsb=0) == WS


def test_varlen_validation_errors(lib):
    """Packed sequences: the varlen descriptor and its arrays are required,
    and only the two-pass algorithms take them (checked before any launch)."""
    vl = _abi.Varlen(FAKE, FAKE)

    def bwd(algo, varlen):
        c = Call(lib, algo=algo)
        ref = lambda t: ctypes.byref(t) if t is not None else None
        v = c.views
        return lib.isattn_attn_bwd_varlen(ctypes.byref(c.shape), ctypes.byref(varlen) if varlen is not None else None,
                                          ref(v["q"]), ref(v["k"]), ref(v["v"]), ref(v["o"]), ref(v["do"]),
                                          c.lse, None, 0, 0.125, ref(v["dq"]), ref(v["dk"]), ref(v["dv"]), algo,
                                          c.ws, c.ws_bytes, None)
    assert bwd(2, None) == NULL
    assert bwd(0, vl) == UNSUP
    assert bwd(1, vl) == UNSUP
    assert bwd(2, _abi.Varlen(None, FAKE)) == NULL
    assert bwd(3, _abi.Varlen(FAKE, None)) == NULL
    s = shape()
    t = _abi.Tensor(FAKE, 256 * 2 * 128, 2 * 128, 128)
    assert lib.isattn_attn_fwd_varlen(ctypes.byref(s), None, ctypes.byref(t), ctypes.byref(t), ctypes.byref(t),
                                      None, 0, 0.125, ctypes.byref(t), FAKE, None) == NULL
    assert lib.isattn_attn_fwd_varlen(ctypes.byref(s), ctypes.byref(_abi.Varlen(FAKE, None)), ctypes.byref(t),
                                      ctypes.byref(t), ctypes.byref(t), None, 0, 0.125, ctypes.byref(t), FAKE,
                                      None) == NULL
    wsb = lib.isattn_index_to_block_sparse_workspace_bytes(1, 256, 256, 2, 128, 128)
    assert lib.isattn_index_to_block_sparse_varlen(FAKE, 1, None, FAKE, 256, 256, 2, 64, 128, 128, FAKE, FAKE,
                                                   FAKE, FAKE, 8, FAKE, wsb, None) == NULL
    assert lib.isattn_index_to_block_sparse_varlen(FAKE, 1, FAKE, FAKE, 256, 256, 2, 64, 128, 128, FAKE, FAKE,
                                                   FAKE, FAKE, 3, FAKE, wsb, None) == CAP


def test_token_bits_validation_errors(lib):
    """Token-exact masks: the two-pass algorithms only, 16-byte aligned bits;
    the bits converter checks its buffer, pointers and sizes."""
    tok = lambda p: _abi.Mask(1, 128, 128, 2, FAKE, FAKE, FAKE, FAKE, p)
    for algo in (0, 1):
        c = Call(lib, algo=algo); c.mask = tok(FAKE); assert c() == UNSUP
    c = Call(lib, algo=2); c.mask = tok(FAKE + 4); assert c() == STRIDE
    need = 1 * 2 * 2 * 2 * 1024
    call = lambda idx=FAKE, bits=FAKE, words=need, cq=None, ck=None, B=1: lib.isattn_index_to_token_bits(
        idx, B, 256, 256, 2, 64, cq, ck, bits, words, None)
    assert call(words=need - 1) == CAP
    assert call(bits=None) == NULL
    assert call(idx=None) == NULL
    assert call(cq=FAKE) == NULL
    assert call(B=-1) == SHAPE
    assert call(bits=FAKE + 4) == STRIDE


def ws_mask(lib, s, algo, mask=None, causal=0, varlen=0):
    return lib.isattn_attn_bwd_workspace_bytes_mask(ctypes.byref(s), algo, ctypes.byref(mask) if mask else None,
                                                    causal, varlen)


def brute_visible_blocks(Sq, Sk, causal):
    """Blocks of one head with a visible pair (bottom-right causal), by enumeration."""
    n = 0
    for qb in range(-(-Sq // 128)):
        for kb in range(-(-Sk // 128)):
            if not causal:
                n += 1
                continue
            last_row = min(qb * 128 + 127, Sq - 1)
            n += kb * 128 <= last_row + Sk - Sq
    return n


def test_split_ds_workspace_by_kept_blocks(lib):
    """SPLIT_DS sizes its dS store by the kept blocks: R * nnz tiles for a
    block CSR (R query heads per mask head) plus an nnz-entry position map
    and an overflow flag,
    B * Hq * (visible blocks of a head) for dense and causal masks, the whole
    block grid for a dense mask over packed sequences."""
    al = lambda x: (x + 255) // 256 * 256
    tile = 128 * 128 * 2
    for (Sq, Sk) in ((300, 200), (200, 300), (1024, 1024), (1000, 130), (130, 1000), (128, 4096), (257, 129)):
        s = shape(B=2, Sq=Sq, Sk=Sk, Hq=4, Hk=2)
        fixed = ws_bytes(lib, s, 2)
        nq, nk = -(-Sq // 128), -(-Sk // 128)
        for causal in (0, 1):
            vis = brute_visible_blocks(Sq, Sk, causal)
            assert ws_mask(lib, s, 3, None, causal) == fixed + al(2 * 4 * vis * tile), (Sq, Sk, causal)
            assert ws_mask(lib, s, 3, None, causal, varlen=1) == fixed + al(2 * 4 * nq * nk * tile)
            for hm in (1, 2, 4):
                m = _abi.Mask(1, 128, 128, hm, FAKE, FAKE, FAKE, FAKE, None, 5)
                assert ws_mask(lib, s, 3, m, causal) == fixed + al(5 * 4 + 4) + al((4 // hm) * 5 * tile)
                unknown = _abi.Mask(1, 128, 128, hm, FAKE, FAKE, FAKE, FAKE)     # nnz not given: every block
                grid = 2 * hm * nq * nk
                assert ws_mask(lib, s, 3, unknown, causal) == fixed + al(grid * 4 + 4) + al((4 // hm) * grid * tile)
        for algo in (0, 1, 2):                     # the other algorithms do not depend on the mask
            assert ws_mask(lib, s, algo, None, 1) == ws_bytes(lib, s, algo)
    # the benchmark's block-sparse workload: 34,112 kept blocks of 16 mask heads -> 1.12 GB, not 4.3 GB
    s = shape(B=2, Sq=8192, Sk=8192, Hq=16, Hk=16)
    m = _abi.Mask(1, 128, 128, 16, FAKE, FAKE, FAKE, FAKE, None, 34112)
    assert ws_mask(lib, s, 3, m) - ws_bytes(lib, s, 2) == al(34112 * 4 + 4) + 34112 * tile
    # the 32K causal d192 workload: 526,336 visible blocks of 16 heads -> 17.2 GB, not 34.4 GB
    s = shape(B=1, Sq=32768, Sk=32768, Hq=16, Hk=16, Dqk=192, Dv=128)
    assert ws_mask(lib, s, 3, None, 1) - ws_bytes(lib, s, 2) == 526336 * tile
    assert ws_mask(lib, s, 3, _abi.Mask(7, 128, 128, 1, None, None, None, None)) == 0
    assert ws_mask(lib, s, 3, _abi.Mask(1, 128, 128, 3, FAKE, FAKE, FAKE, FAKE)) == 0


def test_split_ds_capacity_checked_before_launch(lib):
    """A workspace holding fewer dS tiles than the mask needs is rejected
    with ISATTN_ERR_CAPACITY before any launch (no GPU here: a call that
    passed every check would fail to launch)."""
    tile = 128 * 128 * 2
    # block CSR, 2 mask heads, 6 kept blocks given by the caller
    m = _abi.Mask(1, 128, 128, 2, FAKE, FAKE, FAKE, FAKE, None, 6)
    c = Call(lib, algo=3, Sq=512, Sk=512)
    exact = ws_mask(lib, c.shape, 3, m)
    c.mask = m
    c.ws_bytes = exact - tile                      # one tile short
    assert c() == CAP
    c.mask = _abi.Mask(1, 128, 128, 2, FAKE, FAKE, FAKE, FAKE, None, 7)   # more blocks than the workspace holds
    c.ws_bytes = exact
    assert c() == CAP
    c.mask = _abi.Mask(1, 128, 128, 2, FAKE, FAKE, FAKE, FAKE)           # count unknown: needs every block
    assert c() == CAP
    # dense causal: every visible block of every head
    c = Call(lib, algo=3, Sq=512, Sk=512)
    c.causal = 1
    c.ws_bytes = ws_mask(lib, c.shape, 3, None, 1) - 1
    assert c() == CAP
    c.ws_bytes = ws_bytes(lib, c.shape, 2) - 1     # not even the fixed part
    assert c() == WS


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """isattn_attn_bwd_noalloc checks the size against its static scratch
    before touching a device: past 64 MiB it returns ISATTN_ERR_SCRATCH."""
    def call(**kw):
        c = Call(lib, algo=2, **kw)
        v = c.views
        return lib.isattn_attn_bwd_noalloc(ctypes.byref(c.shape), ctypes.byref(v["q"]), ctypes.byref(v["k"]),
                                           ctypes.byref(v["v"]), ctypes.byref(v["o"]), ctypes.byref(v["do"]),
                                           c.lse, None, 0, 0.125, ctypes.byref(v["dq"]), ctypes.byref(v["dk"]),
                                           ctypes.byref(v["dv"]), None)
    # delta + lse2 = 8 bytes per padded query row: 8 Mi rows need 64 MiB plus the work order
    assert call(B=1, Sq=1 << 20, Sk=128, Hq=8, Hk=8) == SCRATCH
    assert call(B=4, Sq=1 << 18, Sk=256, Hq=8, Hk=1) == SCRATCH
    # 32K tokens x 16 heads (4.3 MiB) fits; the call then needs a GPU, which this host lacks
    assert call(B=1, Sq=32768, Sk=32768, Hq=16, Hk=16) != SCRATCH
