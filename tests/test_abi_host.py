"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
its host-side index builder matches the oracle's brute-force block lists
bit-exactly, and argument validation rejects bad calls before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

import long_context_sparse_static_amd as lcs
from oracle import (ATTNSINK, BLOCKSPARSE, FULL, SLIDING, block_lists, blocksparse_decode_positions,
                    pattern_lists_for_head, transpose_lists)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sparse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 22
    assert sorted(lcs.EXPORTED) == names
    L = lcs.lib()
    for n in names:
        assert hasattr(L, n), n
    # the shared object itself exports them (nm-free check through dlsym)
    raw = ctypes.CDLL(lcs.LIB_PATH)
    for n in names:
        assert ctypes.cast(getattr(raw, n), ctypes.c_void_p).value


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert lcs.attn_status_str(s)
    assert lcs.attn_status_str(-99) == "unknown status"


# ------------------------------------------------------------------ index
PATTERNS = {
    # (pattern, oracle kind, kwargs, heads, L)
    "attnsink_1k": (lcs.attnsink_pattern(1, 4), ATTNSINK, dict(sink_blocks=1, local_blocks=4), 1, 1024),
    "attnsink_8k": (lcs.attnsink_pattern(1, 64), ATTNSINK, dict(sink_blocks=1, local_blocks=64), 1, 8192),
    "blocksparse_32k": (lcs.blocksparse_pattern(1, 16, 8), BLOCKSPARSE,
                        dict(sink_blocks=1, local_blocks=16, stride=8), 32, 32768),
    "attnsink_64k": (lcs.attnsink_pattern(1, 64), ATTNSINK, dict(sink_blocks=1, local_blocks=64), 1, 65536),
    "attnsink_128k": (lcs.attnsink_pattern(1, 64), ATTNSINK, dict(sink_blocks=1, local_blocks=64), 1, 131072),
    "full_32k": (lcs.full_pattern(), FULL, dict(), 1, 32768),
    "odd_sink2": (lcs.attnsink_pattern(2, 3), ATTNSINK, dict(sink_blocks=2, local_blocks=3), 1, 64 * 37),
    "odd_bs": (lcs.blocksparse_pattern(3, 5, 7), BLOCKSPARSE, dict(sink_blocks=3, local_blocks=5, stride=7), 9, 64 * 50),
    "sliding_4096_sink1": (lcs.sliding_pattern(1, 4096), SLIDING, dict(sink_blocks=1, window_tokens=4096), 1, 65536),
    "sliding_1000": (lcs.sliding_pattern(0, 1000), SLIDING, dict(sink_blocks=0, window_tokens=1000), 1, 64 * 40),
    "sliding_1": (lcs.sliding_pattern(0, 1), SLIDING, dict(sink_blocks=0, window_tokens=1), 1, 64 * 9),
    "sliding_65_sink2": (lcs.sliding_pattern(2, 65), SLIDING, dict(sink_blocks=2, window_tokens=65), 1, 64 * 21),
    "sliding_wide": (lcs.sliding_pattern(1, 10 ** 6), SLIDING, dict(sink_blocks=1, window_tokens=10 ** 6), 1, 64 * 13),
}


@pytest.mark.parametrize("name", list(PATTERNS))
def test_index_matches_oracle_bit_exact(name):
    pat, kind, kw, heads, L = PATTERNS[name]
    nb = L // 64
    ix = lcs.attn_index_build(pat, heads, L, with_csc=True)
    lcs.attn_index_validate(ix)
    for h in range(heads):
        want = block_lists(kind, nb, head=h, **kw)
        base = h * (nb + 1)
        got_rows = np.split(ix.col_idx[ix.row_ptr[base]:ix.row_ptr[base + nb]],
                            ix.row_ptr[base + 1:base + nb] - ix.row_ptr[base])
        assert [r.tolist() for r in got_rows] == want, (name, h)
        cols = transpose_lists(want, nb)
        cbase = h * (nb + 1)
        got_cols = np.split(ix.row_idx[ix.col_ptr[cbase]:ix.col_ptr[cbase + nb]],
                            ix.col_ptr[cbase + 1:cbase + nb] - ix.col_ptr[cbase])
        assert [c.tolist() for c in got_cols] == cols, (name, h)


MIXED = [  # (pattern, oracle kind, kwargs) per head: retrieval / streaming head mix
    (lcs.full_pattern(), FULL, dict()),
    (lcs.attnsink_pattern(1, 4), ATTNSINK, dict(sink_blocks=1, local_blocks=4)),
    (lcs.blocksparse_pattern(1, 3, 4), BLOCKSPARSE, dict(sink_blocks=1, local_blocks=3, stride=4)),
    (lcs.attnsink_pattern(2, 3), ATTNSINK, dict(sink_blocks=2, local_blocks=3)),
    (lcs.full_pattern(), FULL, dict()),
    (lcs.blocksparse_pattern(2, 5, 3), BLOCKSPARSE, dict(sink_blocks=2, local_blocks=5, stride=3)),
]


def test_mixed_index_matches_oracle_bit_exact():
    """Per-head pattern mix: head h's rows and columns are those of its own
    pattern (with stride phase h), bit-exact against the oracle's scan."""
    L = 64 * 37
    nb = L // 64
    pats = [m[0] for m in MIXED]
    ix = lcs.attn_index_build_mixed(pats, L, with_csc=True)
    lcs.attn_index_validate(ix)
    total = 0
    for h, (_, kind, kw) in enumerate(MIXED):
        want = block_lists(kind, nb, head=h, **kw)
        total += sum(len(r) for r in want)
        assert [ix.row(h, i) for i in range(nb)] == want, h
        assert [ix.col(h, j) for j in range(nb)] == transpose_lists(want, nb), h
    assert lcs.attn_index_nnz_mixed(pats, L) == total == ix.nnz


def test_mixed_index_rejects_inconsistent_heads():
    L = 64 * 8
    non_causal = lcs.Pattern(lcs.ATTN_ATTNSINK, 1, 2, causal=False)
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz_mixed([lcs.full_pattern(), non_causal], L)     # causal differs
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz_mixed([lcs.full_pattern(), lcs.Pattern(7)], L)  # unknown kind
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz_mixed([lcs.full_pattern()], 0)                 # empty sequence
    with pytest.raises(lcs.AttnError):                                    # one token window per launch
        lcs.attn_index_nnz_mixed([lcs.full_pattern(), lcs.sliding_pattern(1, 100)], L)


def test_sliding_pattern_rejections():
    L = 64 * 8
    for bad in (lcs.sliding_pattern(1, 0), lcs.sliding_pattern(-1, 64),
                lcs.Pattern(lcs.ATTN_SLIDING, 1, 0, 0, False, window_tokens=64)):
        with pytest.raises(lcs.AttnError):
            lcs.attn_index_nnz(bad, 1, L)


@pytest.mark.parametrize("L", [1, 63, 65, 1000, 64 * 9 + 37])
def test_index_of_ragged_length(L):
    """A sequence whose last block is partial has ceil(L / 64) blocks and the
    same lists as the whole-block length: the oracle's scan over ceil(L/64)."""
    nb = -(-L // 64)
    for pat in (lcs.attnsink_pattern(1, 3), lcs.blocksparse_pattern(1, 2, 3), lcs.full_pattern(),
                lcs.sliding_pattern(1, 100)):
        H = 3 if pat.head_dependent else 1
        ix = lcs.attn_index_build(pat, H, L, with_csc=True)
        assert (ix.n_qblocks, ix.n_kblocks) == (nb, nb)
        lcs.attn_index_validate(ix)
        assert ix.nnz == lcs.attn_index_nnz(pat, H, 64 * nb)
        for h in range(H):
            opat = dict(kind={lcs.ATTN_FULL: FULL, lcs.ATTN_ATTNSINK: ATTNSINK, lcs.ATTN_BLOCKSPARSE: BLOCKSPARSE,
                              lcs.ATTN_SLIDING: SLIDING}[pat.kind], block=64, sink_blocks=pat.sink_blocks,
                        local_blocks=pat.local_blocks, stride=pat.stride, window_tokens=pat.window_tokens)
            want = pattern_lists_for_head(opat, nb, h)
            assert [ix.row(h, i) for i in range(nb)] == want
            assert [ix.col(h, j) for j in range(nb)] == transpose_lists(want, nb)


@pytest.mark.parametrize("L", [64 * 11 + 23, 64 * 40])
def test_patterns_listing_every_causal_block_build_the_full_index(L):
    """A window that covers the sequence, BlockSparse with stride 1 (every
    earlier block strided) and a token window longer than the sequence all
    list every causal block: their CSR and CSC arrays equal the full
    pattern's, head by head."""
    nb = -(-L // 64)
    full = lcs.attn_index_build(lcs.full_pattern(), 1, L, with_csc=True)
    for pat in (lcs.attnsink_pattern(1, nb), lcs.attnsink_pattern(0, nb + 5), lcs.blocksparse_pattern(1, 1, 1),
                lcs.blocksparse_pattern(2, 3, 1), lcs.sliding_pattern(1, L + 64)):
        H = 3 if pat.head_dependent else 1
        ix = lcs.attn_index_build(pat, H, L, with_csc=True)
        assert ix.nnz == H * full.nnz
        for h in range(H):
            assert [ix.row(h, i) for i in range(nb)] == [full.row(0, i) for i in range(nb)]
            assert [ix.col(h, j) for j in range(nb)] == [full.col(0, j) for j in range(nb)]


def test_index_nnz_closed_forms():
    assert lcs.attn_index_nnz(lcs.attnsink_pattern(1, 4), 1, 1024) == 70
    assert lcs.attn_index_nnz(lcs.attnsink_pattern(1, 64), 1, 8192) == 6240
    assert lcs.attn_index_nnz(lcs.attnsink_pattern(1, 64), 1, 65536) == 64480
    assert lcs.attn_index_nnz(lcs.attnsink_pattern(1, 64), 1, 131072) == 131040
    assert lcs.attn_index_nnz(lcs.attnsink_pattern(1, 64), 32, 131072) == 32 * 131040
    assert lcs.attn_index_nnz(lcs.blocksparse_pattern(1, 16, 8), 32, 32768) == 765216
    assert lcs.attn_index_nnz(lcs.full_pattern(), 1, 131072) == 2048 * 2049 // 2


def test_index_rejects_bad_arguments():
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz(lcs.attnsink_pattern(1, 4), 1, 0)             # empty sequence
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz(lcs.attnsink_pattern(1, 0), 1, 1024)          # local < 1
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz(lcs.blocksparse_pattern(1, 4, 0), 1, 1024)    # stride < 1
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz(lcs.Pattern(7), 1, 1024)                      # unknown kind
    with pytest.raises(lcs.AttnError):
        lcs.attn_index_nnz(lcs.attnsink_pattern(1, 4), 0, 1024)          # heads < 1


def _corrupt(ix, field, fn):
    import copy
    bad = copy.deepcopy(ix)
    arr = getattr(bad, field).copy()
    fn(arr)
    setattr(bad, field, arr)
    return bad


@pytest.mark.parametrize("field,fn", [
    ("row_ptr", lambda a: a.__setitem__(3, a[4] + 1)),          # non-monotone
    ("row_ptr", lambda a: a.__setitem__(-1, 10 ** 6)),          # beyond nnz
    ("col_idx", lambda a: a.__setitem__(5, 999)),               # block id out of range
    ("col_idx", lambda a: a.__setitem__(slice(1, 3), a[2:0:-1])),  # unsorted row
    ("row_idx", lambda a: a.__setitem__(7, (a[7] + 1) % 16)),   # CSC not the transpose
    ("col_ptr", lambda a: a.__setitem__(2, a[2] + 1)),          # CSC pointer shifted
])
def test_validate_rejects_malformed_index(field, fn):
    ix = lcs.attn_index_build(lcs.attnsink_pattern(1, 4), 1, 1024)
    lcs.attn_index_validate(ix)
    bad = _corrupt(ix, field, fn)
    with pytest.raises(lcs.AttnError) as e:
        lcs.attn_index_validate(bad)
    assert e.value.status == lcs.ATTN_ERR_BAD_INDEX


def test_layer_map_middle_third():
    m = lcs.attn_layer_map(32, 11, 21)
    assert m.tolist() == [0] * 11 + [1] * 11 + [0] * 10
    assert m.sum() == 11


def test_workspace_sizes():
    assert lcs.attn_workspace_bytes(lcs.ATTN_OP_FWD, lcs.ATTN_BF16, 1, 32, 8192, 128) == 0
    assert lcs.attn_workspace_bytes(lcs.ATTN_OP_BWD, lcs.ATTN_BF16, 1, 32, 65536, 128) == 2 * 32 * 65536 * 4
    ws = lcs.attn_workspace_bytes(lcs.ATTN_OP_FULL_DECODE, lcs.ATTN_BF16, 16, 32, 131073, 128)
    assert ws > 0 and ws % (16 * 32 * 130 * 4) == 0
    ws2 = lcs.attn_workspace_bytes(lcs.ATTN_OP_SPARSE_DECODE, lcs.ATTN_BF16, 16, 32, 4160, 128)
    assert 0 < ws2 <= ws


# --------------------------------------------- validation before any launch
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _fwd(dtype=lcs.ATTN_BF16, B=1, H=2, L=256, d=128, scale=0.1, pattern=None, ix=None,
         q=FAKE, lse=FAKE):
    p = pattern or lcs.attnsink_pattern(1, 2).c_struct()
    if ix is None:
        ix = lcs.attn_index_t(1, L // 64, L // 64, 10, FAKE, FAKE, None, None)
    return lcs.lib().attn_sparse_fwd(dtype, B, H, L, d, scale, ctypes.byref(p), ctypes.byref(ix),
                                     q, FAKE, FAKE, FAKE, lse, None, 0, None)


def test_forward_validation_errors():
    assert _fwd(L=1000) == lcs.ATTN_ERR_INVALID_ARG                   # index of 15 blocks, not ceil(1000/64)
    ragged_ix = lcs.attn_index_t(1, 16, 16, 10, FAKE, FAKE, None, None)
    non_causal = lcs.Pattern(lcs.ATTN_ATTNSINK, 1, 2, causal=False).c_struct()
    assert _fwd(L=1000, ix=ragged_ix, pattern=non_causal) == lcs.ATTN_ERR_UNSUPPORTED   # keys past L
    assert _fwd(B=0) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(H=0) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(L=0) == lcs.ATTN_ERR_INVALID_ARG                      # empty sequence
    assert _fwd(L=-64) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(scale=0.0) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(scale=float("nan")) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(q=None) == lcs.ATTN_ERR_INVALID_ARG
    assert _fwd(d=96) == lcs.ATTN_ERR_UNSUPPORTED
    assert _fwd(dtype=7) == lcs.ATTN_ERR_UNSUPPORTED
    bad_blocks = lcs.attn_index_t(1, 3, 4, 10, FAKE, FAKE, None, None)
    assert _fwd(ix=bad_blocks) == lcs.ATTN_ERR_INVALID_ARG           # index shape vs L
    bad_heads = lcs.attn_index_t(3, 4, 4, 10, FAKE, FAKE, None, None)
    assert _fwd(ix=bad_heads) == lcs.ATTN_ERR_INVALID_ARG            # n_heads not 1 or H
    p = lcs.attn_pattern_t(1, 32, 1, 2, 0, 1)
    assert _fwd(pattern=p) == lcs.ATTN_ERR_INVALID_ARG               # block != 64
    # one key block past the bf16 path's LDS bitmap limit (4,161,536 tokens at
    # d = 128): rejected before any launch
    assert _fwd(B=1, H=1, L=4161536 + 64) == lcs.ATTN_ERR_UNSUPPORTED


def test_backward_validation_errors():
    L_ = lcs.lib()
    p = lcs.attnsink_pattern(1, 2).c_struct()
    no_csc = lcs.attn_index_t(1, 4, 4, 10, FAKE, FAKE, None, None)
    csc = lcs.attn_index_t(1, 4, 4, 10, FAKE, FAKE, FAKE, FAKE)
    args = lambda ix, dtype=lcs.ATTN_BF16, ws=FAKE, wsb=1 << 20: (
        dtype, 1, 2, 256, 128, 0.1, ctypes.byref(p), ctypes.byref(ix), FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert L_.attn_sparse_bwd(*args(no_csc)) == lcs.ATTN_ERR_INVALID_ARG
    assert L_.attn_sparse_bwd(*args(csc, dtype=lcs.ATTN_F32)) == lcs.ATTN_ERR_UNSUPPORTED
    assert L_.attn_sparse_bwd(*args(csc, ws=None)) == lcs.ATTN_ERR_WORKSPACE
    assert L_.attn_sparse_bwd(*args(csc, wsb=100)) == lcs.ATTN_ERR_WORKSPACE


def test_decode_validation_errors():
    L_ = lcs.lib()
    base = lambda **kw: dict(dtype=lcs.ATTN_BF16, B=2, H=4, d=128, scale=0.1, sink=64, window=4096,
                             pos=FAKE, ws=FAKE, wsb=1 << 30) | kw
    def sp(**kw):
        a = base(**kw)
        return L_.attn_sparse_decode(a["dtype"], a["B"], a["H"], a["d"], a["scale"], a["sink"],
                                     a["window"], a["pos"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, a["ws"], a["wsb"], None)
    assert sp(window=0) == lcs.ATTN_ERR_INVALID_ARG
    assert sp(sink=-1) == lcs.ATTN_ERR_INVALID_ARG
    assert sp(pos=None) == lcs.ATTN_ERR_INVALID_ARG
    assert sp(d=80) == lcs.ATTN_ERR_UNSUPPORTED
    assert sp(dtype=lcs.ATTN_F32) == lcs.ATTN_ERR_UNSUPPORTED
    assert sp(ws=None) == lcs.ATTN_ERR_WORKSPACE
    assert sp(wsb=16) == lcs.ATTN_ERR_WORKSPACE

    def fd(cap=1000, max_pos=999, wsb=1 << 30):
        return L_.attn_full_decode(lcs.ATTN_BF16, 2, 4, 128, 0.1, cap, max_pos, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, None)
    assert fd(max_pos=1000) == lcs.ATTN_ERR_INVALID_ARG       # max_pos >= capacity
    assert fd(max_pos=-1) == lcs.ATTN_ERR_INVALID_ARG
    assert fd(wsb=8) == lcs.ATTN_ERR_WORKSPACE

    def fdn(cap=1000, max_pos=999, B=2, d=128):
        return L_.attn_full_decode_noalloc(lcs.ATTN_BF16, B, 4, d, 0.1, cap, max_pos, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    # argument errors come back before the fixed scratch is looked up (no GPU here)
    assert fdn(max_pos=1000) == lcs.ATTN_ERR_INVALID_ARG
    assert fdn(B=0) == lcs.ATTN_ERR_INVALID_ARG
    assert fdn(d=80) == lcs.ATTN_ERR_UNSUPPORTED

    rf = L_.attn_ring_fill
    assert rf(lcs.ATTN_BF16, 1, 1, 128, 64, 0, FAKE, FAKE, FAKE, 10, FAKE, FAKE, None) == lcs.ATTN_ERR_INVALID_ARG
    assert rf(lcs.ATTN_BF16, 1, 1, 100, 64, 64, FAKE, FAKE, FAKE, 10, FAKE, FAKE, None) == lcs.ATTN_ERR_UNSUPPORTED


def test_blocksparse_decode_validation_errors():
    """The compacted-cache decode and its fill reject a pattern that is not
    BlockSparse with 64-token blocks, a negative strided capacity, a cache
    beyond int32 slots, missing pointers, and a short workspace."""
    L_ = lcs.lib()
    good = lcs.blocksparse_pattern(1, 16, 8)

    def pat(kind=lcs.ATTN_BLOCKSPARSE, block=64, sink=1, local=16, stride=8):
        p = good.c_struct()
        p.kind, p.block, p.sink_blocks, p.local_blocks, p.stride = kind, block, sink, local, stride
        return p

    def dec(p=None, cap=256, B=2, H=4, d=128, scale=0.1, pos=FAKE, dtype=lcs.ATTN_BF16, ws=FAKE,
            wsb=1 << 30):
        p = pat() if p is None else p
        return L_.attn_blocksparse_decode(dtype, B, H, d, scale, ctypes.byref(p), cap, pos, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert dec(p=pat(kind=lcs.ATTN_ATTNSINK)) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(p=pat(block=32)) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(p=pat(local=0)) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(p=pat(stride=0)) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(p=pat(sink=-1)) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(cap=-1) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(cap=1 << 25) == lcs.ATTN_ERR_INVALID_ARG           # more than 2^31 slots
    assert dec(scale=0.0) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(scale=float("nan")) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(pos=None) == lcs.ATTN_ERR_INVALID_ARG
    assert dec(B=300, H=300) == lcs.ATTN_ERR_INVALID_ARG           # B*H beyond the grid
    assert dec(d=96) == lcs.ATTN_ERR_UNSUPPORTED
    assert dec(dtype=lcs.ATTN_F32) == lcs.ATTN_ERR_UNSUPPORTED
    assert dec(ws=None) == lcs.ATTN_ERR_WORKSPACE
    assert dec(wsb=16) == lcs.ATTN_ERR_WORKSPACE
    need = lcs.attn_workspace_bytes(lcs.ATTN_OP_BLOCKSPARSE_DECODE, lcs.ATTN_BF16, 2, 4,
                                    64 * (1 + 16 + 256), 128)
    assert dec(wsb=need - 1) == lcs.ATTN_ERR_WORKSPACE

    def fill(p=None, cap=256, src_len=100, ln=FAKE, d=128, dtype=lcs.ATTN_BF16):
        p = pat() if p is None else p
        return L_.attn_blocksparse_cache_fill(dtype, 2, 4, d, ctypes.byref(p), cap, ln, FAKE, FAKE,
                                              src_len, FAKE, FAKE, None)
    assert fill(p=pat(kind=lcs.ATTN_FULL)) == lcs.ATTN_ERR_INVALID_ARG
    assert fill(cap=-2) == lcs.ATTN_ERR_INVALID_ARG
    assert fill(src_len=-1) == lcs.ATTN_ERR_INVALID_ARG
    assert fill(ln=None) == lcs.ATTN_ERR_INVALID_ARG
    assert fill(d=80) == lcs.ATTN_ERR_UNSUPPORTED
    assert fill(dtype=lcs.ATTN_F32) == lcs.ATTN_ERR_UNSUPPORTED


def test_strided_validation_errors():
    """Strides that are not whole 16-byte vectors, negative strides, a token
    stride beyond 64-row int32 offsets and a misaligned base are rejected
    before any launch."""
    L_ = lcs.lib()
    p = lcs.attnsink_pattern(1, 2).c_struct()
    ix = lcs.attn_index_t(1, 4, 4, 10, FAKE, FAKE, None, None)
    good = lcs.attn_strides_t(2 * 256 * 128, 256 * 128, 128)

    def fwd(qs=good, q=FAKE, dtype=lcs.ATTN_BF16):
        return L_.attn_sparse_fwd_strided(dtype, 1, 2, 256, 128, 0.1, ctypes.byref(p), ctypes.byref(ix),
                                          q, ctypes.byref(qs), FAKE, ctypes.byref(good), FAKE,
                                          ctypes.byref(good), FAKE, ctypes.byref(good), FAKE, None, 0,
                                          None)
    assert fwd(qs=lcs.attn_strides_t(65536, 32768, 132)) == lcs.ATTN_ERR_INVALID_ARG   # 264 B rows
    assert fwd(qs=lcs.attn_strides_t(65536, -32768, 128)) == lcs.ATTN_ERR_INVALID_ARG
    assert fwd(qs=lcs.attn_strides_t(65536, 32768, 1 << 25)) == lcs.ATTN_ERR_INVALID_ARG
    assert fwd(q=ctypes.c_void_p(0x1008)) == lcs.ATTN_ERR_INVALID_ARG                  # 8-byte aligned
    assert fwd(qs=lcs.attn_strides_t(65536, 32768, 130), dtype=lcs.ATTN_F32) == lcs.ATTN_ERR_INVALID_ARG
    csc = lcs.attn_index_t(1, 4, 4, 10, FAKE, FAKE, FAKE, FAKE)
    bad = lcs.attn_strides_t(0, 0, 12)
    g = ctypes.byref(good)
    assert L_.attn_sparse_bwd_strided(lcs.ATTN_BF16, 1, 2, 256, 128, 0.1, ctypes.byref(p),
                                      ctypes.byref(csc), FAKE, g, FAKE, g, FAKE, g, FAKE, g, FAKE,
                                      FAKE, g, FAKE, g, FAKE, ctypes.byref(bad), FAKE, g, FAKE,
                                      1 << 20, None) == lcs.ATTN_ERR_INVALID_ARG


def test_sliding_forward_requires_causal():
    p = lcs.Pattern(lcs.ATTN_SLIDING, 1, 0, 0, False, window_tokens=100).c_struct()
    assert _fwd(pattern=p) == lcs.ATTN_ERR_INVALID_ARG
    p = lcs.sliding_pattern(1, 0).c_struct()
    assert _fwd(pattern=p) == lcs.ATTN_ERR_INVALID_ARG


def test_paged_validation_errors():
    L_ = lcs.lib()

    def pd(n_pages=10, max_pages=4, table=FAKE, max_pos=255, wsb=1 << 30):
        return L_.attn_paged_decode(lcs.ATTN_BF16, 2, 4, 128, 0.1, n_pages, max_pages, table, max_pos,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, None)
    assert pd(n_pages=0) == lcs.ATTN_ERR_INVALID_ARG
    assert pd(table=None) == lcs.ATTN_ERR_INVALID_ARG
    assert pd(max_pos=256) == lcs.ATTN_ERR_INVALID_ARG          # beyond 64 * max_pages - 1
    assert pd(wsb=8) == lcs.ATTN_ERR_WORKSPACE
    pf = L_.attn_paged_cache_fill
    assert pf(lcs.ATTN_BF16, 2, 4, 128, 10, 0, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, None) == lcs.ATTN_ERR_INVALID_ARG
    assert pf(lcs.ATTN_BF16, 2, 4, 96, 10, 4, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, None) == lcs.ATTN_ERR_UNSUPPORTED


# ------------------------------------------------------ BlockSparse cache sizing
@pytest.mark.parametrize("s,w,stride,max_tokens", [(1, 16, 8, 64 * 90 + 5), (1, 16, 8, 64 * 17), (2, 3, 5, 64 * 40),
                                                   (0, 1, 1, 64 * 12 + 1), (3, 5, 7, 64 * 33 - 1),
                                                   (1, 4, 2, 10)])
def test_blocksparse_cache_sizing_against_oracle(s, w, stride, max_tokens):
    """The strided capacity is the most strided blocks (read, not sink, not
    in the token's own window) that the oracle's decode row of any position
    t < max_tokens holds, over every stride phase; the slot count is the
    cache's S."""
    pat = lcs.blocksparse_pattern(s, w, stride)
    opat = dict(kind=BLOCKSPARSE, block=64, sink_blocks=s, local_blocks=w, stride=stride, causal=True)
    most = 0
    for h in range(stride):
        for t in list(range(0, max_tokens, 61)) + [max_tokens - 1]:
            i = t // 64
            blocks = set(blocksparse_decode_positions(t, opat, h) // 64)
            most = max(most, len([j for j in blocks if j >= s and j < i - w + 1]))
    cap = lcs.attn_blocksparse_strided_capacity(pat, max_tokens)
    assert cap == most
    assert lcs.attn_blocksparse_cache_slots(pat, cap) == 64 * (s + w + cap)


def test_blocksparse_cache_sizing_workload():
    """128K BlockSparse (sink 1, local 16, stride 8) decode at t = 131072:
    254 strided blocks, 17,344 slots."""
    pat = lcs.blocksparse_pattern(1, 16, 8)
    assert lcs.attn_blocksparse_strided_capacity(pat, 131073) == 254
    assert lcs.attn_blocksparse_cache_slots(pat, 254) == 17344


def test_blocksparse_cache_sizing_rejections():
    L = lcs.lib()
    out32, out64 = ctypes.c_int32(-7), ctypes.c_int64(-7)
    good = lcs.blocksparse_pattern(1, 16, 8).c_struct()
    for bad in (lcs.attnsink_pattern(1, 4).c_struct(), lcs.blocksparse_pattern(1, 0, 8).c_struct(),
                lcs.blocksparse_pattern(1, 4, 0).c_struct(), lcs.blocksparse_pattern(-1, 4, 8).c_struct()):
        assert L.attn_blocksparse_strided_capacity(ctypes.byref(bad), 1000, ctypes.byref(out32)) == lcs.ATTN_ERR_INVALID_ARG
        assert L.attn_blocksparse_cache_slots(ctypes.byref(bad), 3, ctypes.byref(out64)) == lcs.ATTN_ERR_INVALID_ARG
    assert L.attn_blocksparse_strided_capacity(ctypes.byref(good), 0, ctypes.byref(out32)) == lcs.ATTN_ERR_INVALID_ARG
    assert L.attn_blocksparse_strided_capacity(ctypes.byref(good), 1000, None) == lcs.ATTN_ERR_INVALID_ARG
    assert L.attn_blocksparse_cache_slots(ctypes.byref(good), -1, ctypes.byref(out64)) == lcs.ATTN_ERR_INVALID_ARG
    assert L.attn_blocksparse_cache_slots(ctypes.byref(good), 2 ** 31 - 1, ctypes.byref(out64)) == lcs.ATTN_ERR_UNSUPPORTED
    assert out32.value == -7 and out64.value == -7          # nothing written on an error


def _random_pattern(rng):
    kind = int(rng.integers(0, 4))
    if kind == 0:
        return lcs.full_pattern()
    if kind == 1:
        return lcs.attnsink_pattern(int(rng.integers(0, 5)), int(rng.integers(1, 21)))
    if kind == 2:
        return lcs.blocksparse_pattern(int(rng.integers(0, 5)), int(rng.integers(1, 21)), int(rng.integers(1, 10)))
    return lcs.sliding_pattern(int(rng.integers(0, 4)), int(rng.integers(1, 3000)))


@pytest.mark.parametrize("seed", range(4))
def test_index_of_random_patterns_matches_oracle(seed):
    """Seeded random pattern parameters (sink, local, stride, token window),
    head counts and lengths, whole and ragged: the builder's CSR and CSC equal
    the oracle's brute-force lists, and nnz its count."""
    rng = np.random.default_rng(7100 + seed)
    kinds = {lcs.ATTN_FULL: FULL, lcs.ATTN_ATTNSINK: ATTNSINK, lcs.ATTN_BLOCKSPARSE: BLOCKSPARSE,
             lcs.ATTN_SLIDING: SLIDING}
    for _ in range(15):
        pat = _random_pattern(rng)
        L = int(rng.integers(1, 64 * 60))
        nb = -(-L // 64)
        H = int(rng.integers(1, 6)) if pat.head_dependent else 1
        ix = lcs.attn_index_build(pat, H, L, with_csc=True)
        lcs.attn_index_validate(ix)
        opat = dict(kind=kinds[pat.kind], block=64, sink_blocks=pat.sink_blocks, local_blocks=pat.local_blocks,
                    stride=pat.stride, window_tokens=pat.window_tokens)
        total = 0
        for h in range(H):
            want = pattern_lists_for_head(opat, nb, h)
            total += sum(len(r) for r in want)
            assert [ix.row(h, i) for i in range(nb)] == want, (pat, L, h)
            assert [ix.col(h, j) for j in range(nb)] == transpose_lists(want, nb), (pat, L, h)
        assert ix.nnz == total == lcs.attn_index_nnz(pat, H, L)
