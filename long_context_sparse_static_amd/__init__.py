"""Static block-sparse causal attention for MI355X (gfx950).

Thin ctypes binding over ``libattn_sparse.so`` (C ABI in
``include/attn_sparse.h``).  Every function here only checks and marshals
arguments -- torch tensors to raw device pointers plus the current HIP stream
-- and calls the C entry point of the same name; all arithmetic runs in the
library's HIP kernels.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

The method is LongGen's hybrid long-context attention: sink + window
(AttnSink) and sink + window + strided (BlockSparse) static block patterns in
the sparse layers, full attention in the middle third of the layers (mlsanity
index page "A Little Goes a Long Way...", "Abstract (arXiv)"; atlas.scime.ai
summary, "Approach").
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_sparse.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_BAD_INDEX = -3
ATTN_ERR_WORKSPACE = -4
ATTN_ERR_HIP = -5

ATTN_F32 = 0
ATTN_BF16 = 1

ATTN_FULL = 0
ATTN_ATTNSINK = 1
ATTN_BLOCKSPARSE = 2
ATTN_SLIDING = 3

ATTN_OP_FWD = 0
ATTN_OP_BWD = 1
ATTN_OP_SPARSE_DECODE = 2
ATTN_OP_FULL_DECODE = 3
ATTN_OP_BLOCKSPARSE_DECODE = 4

BLOCK = 64

# Every symbol include/attn_sparse.h declares.
EXPORTED = (
    "attn_status_str", "attn_index_nnz", "attn_index_build", "attn_index_nnz_mixed",
    "attn_index_build_mixed", "attn_index_validate",
    "attn_layer_map", "attn_workspace_bytes", "attn_sparse_fwd", "attn_sparse_bwd",
    "attn_sparse_decode", "attn_full_decode", "attn_ring_fill", "attn_blocksparse_decode",
    "attn_blocksparse_cache_fill", "attn_paged_decode", "attn_paged_cache_fill",
    "attn_sparse_fwd_strided", "attn_sparse_bwd_strided", "attn_blocksparse_strided_capacity",
    "attn_blocksparse_cache_slots", "attn_full_decode_noalloc",
)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_str(status)} ({status})")


class attn_pattern_t(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("block", ctypes.c_int32),
                ("sink_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
                ("stride", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32)]


class attn_strides_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


class attn_index_t(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_qblocks", ctypes.c_int32),
                ("n_kblocks", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("col_ptr", ctypes.c_void_p), ("row_idx", ctypes.c_void_p)]


_lib_handle = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m long_context_sparse_static_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz, f32 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_float)
        P = ctypes.POINTER
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_status_str.argtypes = [i32]
        L.attn_index_nnz.restype = i32
        L.attn_index_nnz.argtypes = [P(attn_pattern_t), i32, i64, P(i64)]
        L.attn_index_build.restype = i32
        L.attn_index_build.argtypes = [P(attn_pattern_t), i32, i64, vp, vp, vp, vp]
        L.attn_index_nnz_mixed.restype = i32
        L.attn_index_nnz_mixed.argtypes = [P(attn_pattern_t), i32, i64, P(i64)]
        L.attn_index_build_mixed.restype = i32
        L.attn_index_build_mixed.argtypes = [P(attn_pattern_t), i32, i64, vp, vp, vp, vp]
        L.attn_index_validate.restype = i32
        L.attn_index_validate.argtypes = [P(attn_index_t)]
        L.attn_layer_map.restype = i32
        L.attn_layer_map.argtypes = [i32, i32, i32, vp]
        L.attn_workspace_bytes.restype = sz
        L.attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i64, i32]
        L.attn_sparse_fwd.restype = i32
        L.attn_sparse_fwd.argtypes = [i32, i32, i32, i64, i32, f32, P(attn_pattern_t),
                                      P(attn_index_t), vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_sparse_bwd.restype = i32
        L.attn_sparse_bwd.argtypes = [i32, i32, i32, i64, i32, f32, P(attn_pattern_t),
                                      P(attn_index_t), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        L.attn_sparse_decode.restype = i32
        L.attn_sparse_decode.argtypes = [i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, sz, vp]
        L.attn_full_decode.restype = i32
        L.attn_full_decode.argtypes = [i32, i32, i32, i32, f32, i64, i64, vp, vp, vp, vp,
                                       vp, vp, vp, vp, vp, sz, vp]
        L.attn_full_decode_noalloc.restype = i32
        L.attn_full_decode_noalloc.argtypes = [i32, i32, i32, i32, f32, i64, i64, vp, vp, vp, vp,
                                               vp, vp, vp, vp, vp]
        L.attn_ring_fill.restype = i32
        L.attn_ring_fill.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp,
                                     vp]
        L.attn_blocksparse_decode.restype = i32
        L.attn_blocksparse_decode.argtypes = [i32, i32, i32, i32, f32, P(attn_pattern_t), i32, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_blocksparse_strided_capacity.restype = i32
        L.attn_blocksparse_strided_capacity.argtypes = [P(attn_pattern_t), i64, P(i32)]
        L.attn_blocksparse_cache_slots.restype = i32
        L.attn_blocksparse_cache_slots.argtypes = [P(attn_pattern_t), i32, P(i64)]
        L.attn_blocksparse_cache_fill.restype = i32
        L.attn_blocksparse_cache_fill.argtypes = [i32, i32, i32, i32, P(attn_pattern_t), i32, vp,
                                                  vp, vp, i64, vp, vp, vp]
        S = P(attn_strides_t)
        L.attn_sparse_fwd_strided.restype = i32
        L.attn_sparse_fwd_strided.argtypes = [i32, i32, i32, i64, i32, f32, P(attn_pattern_t),
                                              P(attn_index_t), vp, S, vp, S, vp, S, vp, S, vp, vp,
                                              sz, vp]
        L.attn_sparse_bwd_strided.restype = i32
        L.attn_sparse_bwd_strided.argtypes = [i32, i32, i32, i64, i32, f32, P(attn_pattern_t),
                                              P(attn_index_t), vp, S, vp, S, vp, S, vp, S, vp, vp,
                                              S, vp, S, vp, S, vp, S, vp, sz, vp]
        L.attn_paged_decode.restype = i32
        L.attn_paged_decode.argtypes = [i32, i32, i32, i32, f32, i32, i32, vp, i64, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_paged_cache_fill.restype = i32
        L.attn_paged_cache_fill.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i64,
                                            vp, vp, vp]
        _lib_handle = L
    return _lib_handle


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


# ----------------------------------------------------------------------------
# Patterns and the block index (host helpers)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Pattern:
    """Static block pattern (see attn_pattern_t)."""
    kind: int
    sink_blocks: int = 0
    local_blocks: int = 0
    stride: int = 0
    causal: bool = True
    block: int = BLOCK
    window_tokens: int = 0

    def c_struct(self) -> attn_pattern_t:
        return attn_pattern_t(self.kind, self.block, self.sink_blocks, self.local_blocks,
                              self.stride, 1 if self.causal else 0, self.window_tokens)

    @property
    def head_dependent(self) -> bool:
        return self.kind == ATTN_BLOCKSPARSE


def full_pattern(causal: bool = True) -> Pattern:
    return Pattern(ATTN_FULL, causal=causal)


def attnsink_pattern(sink_blocks: int, local_blocks: int, causal: bool = True) -> Pattern:
    return Pattern(ATTN_ATTNSINK, sink_blocks, local_blocks, 0, causal)


def blocksparse_pattern(sink_blocks: int, local_blocks: int, stride: int,
                        causal: bool = True) -> Pattern:
    return Pattern(ATTN_BLOCKSPARSE, sink_blocks, local_blocks, stride, causal)


def sliding_pattern(sink_blocks: int, window_tokens: int) -> Pattern:
    """Token-granular window of ``window_tokens`` tokens (the query and the
    window_tokens - 1 before it) plus ``sink_blocks`` sink blocks; 0 sink
    blocks is plain sliding-window attention."""
    return Pattern(ATTN_SLIDING, sink_blocks, 0, 0, True, window_tokens=window_tokens)


def attn_index_nnz(pattern: Pattern, n_heads: int, L: int) -> int:
    out = ctypes.c_int64(0)
    p = pattern.c_struct()
    _check(lib().attn_index_nnz(ctypes.byref(p), n_heads, L, ctypes.byref(out)), "attn_index_nnz")
    return out.value


@dataclass
class HostIndex:
    n_heads: int
    n_qblocks: int
    n_kblocks: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    col_ptr: np.ndarray | None
    row_idx: np.ndarray | None

    @property
    def nnz(self) -> int:
        return int(self.col_idx.size)

    def c_struct(self) -> attn_index_t:
        ptr = lambda a: None if a is None else a.ctypes.data
        return attn_index_t(self.n_heads, self.n_qblocks, self.n_kblocks, self.nnz,
                            ptr(self.row_ptr), ptr(self.col_idx), ptr(self.col_ptr),
                            ptr(self.row_idx))

    def row(self, head: int, i: int) -> list:
        base = head * (self.n_qblocks + 1)
        return self.col_idx[self.row_ptr[base + i]:self.row_ptr[base + i + 1]].tolist()

    def col(self, head: int, j: int) -> list:
        base = head * (self.n_kblocks + 1)
        return self.row_idx[self.col_ptr[base + j]:self.col_ptr[base + j + 1]].tolist()


def attn_index_build(pattern: Pattern, n_heads: int, L: int, with_csc: bool = True) -> HostIndex:
    """Builds the CSR (and CSC) of ``pattern`` on the host (C++ builder)."""
    nnz = attn_index_nnz(pattern, n_heads, L)
    nb = -(-L // pattern.block)   # the last block may be partial
    row_ptr = np.zeros(n_heads * (nb + 1), dtype=np.int32)
    col_idx = np.zeros(max(nnz, 1), dtype=np.int32)[:nnz]
    col_ptr = np.zeros(n_heads * (nb + 1), dtype=np.int32) if with_csc else None
    row_idx = np.zeros(max(nnz, 1), dtype=np.int32)[:nnz] if with_csc else None
    p = pattern.c_struct()
    ptr = lambda a: None if a is None else a.ctypes.data
    _check(lib().attn_index_build(ctypes.byref(p), n_heads, L, ptr(row_ptr), ptr(col_idx),
                                  ptr(col_ptr), ptr(row_idx)), "attn_index_build")
    return HostIndex(n_heads, nb, nb, row_ptr, col_idx, col_ptr, row_idx)


def attn_index_validate(index: HostIndex) -> None:
    s = index.c_struct()
    _check(lib().attn_index_validate(ctypes.byref(s)), "attn_index_validate")


def attn_layer_map(n_layers: int, full_first: int, full_last: int) -> np.ndarray:
    out = np.zeros(n_layers, dtype=np.uint8)
    _check(lib().attn_layer_map(n_layers, full_first, full_last, out.ctypes.data),
           "attn_layer_map")
    return out


def attn_workspace_bytes(op: int, dtype: int, B: int, H: int, L_or_cap: int, d: int) -> int:
    return int(lib().attn_workspace_bytes(op, dtype, B, H, L_or_cap, d))


class DeviceIndex:
    """A HostIndex uploaded to device memory (torch int32 tensors)."""

    def __init__(self, host: HostIndex, device):
        import torch
        self.host = host
        up = lambda a: None if a is None else torch.from_numpy(a).to(device)
        self.row_ptr = up(host.row_ptr)
        self.col_idx = up(host.col_idx) if host.nnz else torch.zeros(1, dtype=torch.int32,
                                                                      device=device)
        self.col_ptr = up(host.col_ptr)
        self.row_idx = up(host.row_idx) if host.row_idx is not None and host.nnz else (
            None if host.row_idx is None else torch.zeros(1, dtype=torch.int32, device=device))

    def c_struct(self) -> attn_index_t:
        ptr = lambda t: None if t is None else t.data_ptr()
        h = self.host
        return attn_index_t(h.n_heads, h.n_qblocks, h.n_kblocks, h.nnz, ptr(self.row_ptr),
                            ptr(self.col_idx), ptr(self.col_ptr), ptr(self.row_idx))


def build_device_index(pattern: Pattern, H: int, L: int, device, with_csc: bool = True) -> DeviceIndex:
    n_heads = H if pattern.head_dependent else 1
    return DeviceIndex(attn_index_build(pattern, n_heads, L, with_csc), device)


def _pattern_array(patterns):
    arr = (attn_pattern_t * len(patterns))()
    for h, pat in enumerate(patterns):
        arr[h] = pat.c_struct()
    return arr


def attn_index_nnz_mixed(patterns, L: int) -> int:
    """Entries of a per-head mix of patterns (head h follows patterns[h])."""
    out = ctypes.c_int64(0)
    arr = _pattern_array(patterns)
    _check(lib().attn_index_nnz_mixed(arr, len(patterns), L, ctypes.byref(out)),
           "attn_index_nnz_mixed")
    return out.value


def attn_index_build_mixed(patterns, L: int, with_csc: bool = True) -> HostIndex:
    """CSR (and CSC) of a per-head mix of patterns, built on the host."""
    H = len(patterns)
    nnz = attn_index_nnz_mixed(patterns, L)
    nb = -(-L // patterns[0].block)
    row_ptr = np.zeros(H * (nb + 1), dtype=np.int32)
    col_idx = np.zeros(max(nnz, 1), dtype=np.int32)[:nnz]
    col_ptr = np.zeros(H * (nb + 1), dtype=np.int32) if with_csc else None
    row_idx = np.zeros(max(nnz, 1), dtype=np.int32)[:nnz] if with_csc else None
    arr = _pattern_array(patterns)
    ptr = lambda a: None if a is None else a.ctypes.data
    _check(lib().attn_index_build_mixed(arr, H, L, ptr(row_ptr), ptr(col_idx), ptr(col_ptr),
                                        ptr(row_idx)), "attn_index_build_mixed")
    return HostIndex(H, nb, nb, row_ptr, col_idx, col_ptr, row_idx)


def build_device_index_mixed(patterns, L: int, device, with_csc: bool = True) -> DeviceIndex:
    return DeviceIndex(attn_index_build_mixed(patterns, L, with_csc), device)


# ----------------------------------------------------------------------------
# Device operations
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, shape=None, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def attn_sparse_fwd(q, k, v, index: DeviceIndex, pattern: Pattern, scale=None, o=None, lse=None):
    """Prefill forward.  q/k/v [B,H,L,d] (bf16 or fp32) -> (o, lse)."""
    torch = _torch()
    B, H, L, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    args = [_dev(x, n, q.shape, q.dtype, q.device) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = _dev(lse, "lse", (B, H, L), torch.float32, q.device)
    p = pattern.c_struct()
    ix = index.c_struct()
    _check(lib().attn_sparse_fwd(_dtype_code(q), B, H, L, d, scale, ctypes.byref(p),
                                 ctypes.byref(ix), *args, lp, None, 0, _stream()),
           "attn_sparse_fwd")
    return o, lse


def attn_sparse_bwd(q, k, v, o, lse, dout, index: DeviceIndex, pattern: Pattern, scale=None,
                    dq=None, dk=None, dv=None, workspace=None):
    """Backward.  Returns (dq, dk, dv) for loss gradients ``dout``."""
    torch = _torch()
    B, H, L, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    need = attn_workspace_bytes(ATTN_OP_BWD, _dtype_code(q), B, H, L, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ptrs = [_dev(x, n, q.shape, q.dtype, q.device) for x, n in
            ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = _dev(lse, "lse", (B, H, L), torch.float32, q.device)
    dp = _dev(dout, "dout", q.shape, q.dtype, q.device)
    outs = [_dev(x, n, q.shape, q.dtype, q.device) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    wp = _dev(workspace, "workspace", device=q.device)
    p = pattern.c_struct()
    ix = index.c_struct()
    _check(lib().attn_sparse_bwd(_dtype_code(q), B, H, L, d, scale, ctypes.byref(p),
                                 ctypes.byref(ix), *ptrs, lp, dp, *outs, wp,
                                 workspace.numel() * workspace.element_size(), _stream()),
           "attn_sparse_bwd")
    return dq, dk, dv


def _view(t, name, shape, dtype, device):
    """Pointer and element strides of a [B,H,L,d]-indexed device tensor view
    whose last dimension is contiguous (any strides otherwise)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be {dtype} on {device}")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")
    return t.data_ptr(), attn_strides_t(t.stride(0), t.stride(1), t.stride(2))


def attn_sparse_fwd_strided(q, k, v, index: DeviceIndex, pattern: Pattern, scale=None, o=None,
                            lse=None):
    """Prefill forward on [B,H,L,d]-indexed views with any strides (for
    example ``x.transpose(1, 2)`` of [B,L,H,d] activations, or slices of a
    fused QKV projection).  ``o`` defaults to ``empty_like(q)``."""
    torch = _torch()
    B, H, L, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    views = [_view(x, n, q.shape, q.dtype, q.device) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = _dev(lse, "lse", (B, H, L), torch.float32, q.device)
    args = [a for ptr, st in views for a in (ptr, ctypes.byref(st))]
    p = pattern.c_struct()
    ix = index.c_struct()
    _check(lib().attn_sparse_fwd_strided(_dtype_code(q), B, H, L, d, scale, ctypes.byref(p),
                                         ctypes.byref(ix), *args, lp, None, 0, _stream()),
           "attn_sparse_fwd_strided")
    return o, lse


def attn_sparse_bwd_strided(q, k, v, o, lse, dout, index: DeviceIndex, pattern: Pattern,
                            scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward on [B,H,L,d]-indexed views with any strides; the gradients
    default to ``empty_like`` of q, k and v."""
    torch = _torch()
    B, H, L, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_workspace_bytes(ATTN_OP_BWD, _dtype_code(q), B, H, L, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    v4 = [_view(x, n, q.shape, q.dtype, q.device) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = _dev(lse, "lse", (B, H, L), torch.float32, q.device)
    vd = _view(dout, "dout", q.shape, q.dtype, q.device)
    vg = [_view(x, n, q.shape, q.dtype, q.device) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    wp = _dev(workspace, "workspace", device=q.device)
    flat = lambda vs: [a for ptr, st in vs for a in (ptr, ctypes.byref(st))]
    p = pattern.c_struct()
    ix = index.c_struct()
    _check(lib().attn_sparse_bwd_strided(_dtype_code(q), B, H, L, d, scale, ctypes.byref(p),
                                         ctypes.byref(ix), *flat(v4), lp, *flat([vd]), *flat(vg), wp,
                                         workspace.numel() * workspace.element_size(), _stream()),
           "attn_sparse_bwd_strided")
    return dq, dk, dv


def _decode_io(q, k_new, v_new, o, lse):
    torch = _torch()
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError("decode q must be [B,H,1,d]")
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    ptrs = [_dev(x, n, q.shape, q.dtype, q.device) for x, n in
            ((q, "q"), (k_new, "k_new"), (v_new, "v_new"))]
    return B, H, d, o, lse, ptrs


def attn_sparse_decode(q, k_new, v_new, k_cache, v_cache, pos, sink_tokens: int,
                       window_tokens: int, scale=None, o=None, lse=None, workspace=None):
    """Decode one token per sequence against a sink+window ring cache."""
    torch = _torch()
    B, H, d, o, lse, ptrs = _decode_io(q, k_new, v_new, o, lse)
    S = sink_tokens + window_tokens
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kc = _dev(k_cache, "k_cache", (B, H, S, d), q.dtype, q.device)
    vc = _dev(v_cache, "v_cache", (B, H, S, d), q.dtype, q.device)
    pp = _dev(pos, "pos", (B,), torch.int64, q.device)
    need = attn_workspace_bytes(ATTN_OP_SPARSE_DECODE, _dtype_code(q), B, H, S, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace", device=q.device)
    op = _dev(o, "o", q.shape, q.dtype, q.device)
    lp = _dev(lse, "lse", (B, H), torch.float32, q.device)
    _check(lib().attn_sparse_decode(_dtype_code(q), B, H, d, scale, sink_tokens, window_tokens,
                                    pp, *ptrs, kc, vc, op, lp, wp,
                                    workspace.numel() * workspace.element_size(), _stream()),
           "attn_sparse_decode")
    return o, lse


def attn_full_decode(q, k_new, v_new, k_cache, v_cache, pos, max_pos: int, scale=None, o=None,
                     lse=None, workspace=None):
    """Decode one token per sequence against a full cache [B,H,capacity,d]."""
    torch = _torch()
    B, H, d, o, lse, ptrs = _decode_io(q, k_new, v_new, o, lse)
    cap = k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kc = _dev(k_cache, "k_cache", (B, H, cap, d), q.dtype, q.device)
    vc = _dev(v_cache, "v_cache", (B, H, cap, d), q.dtype, q.device)
    pp = _dev(pos, "pos", (B,), torch.int64, q.device)
    need = attn_workspace_bytes(ATTN_OP_FULL_DECODE, _dtype_code(q), B, H, max_pos + 1, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace", device=q.device)
    op = _dev(o, "o", q.shape, q.dtype, q.device)
    lp = _dev(lse, "lse", (B, H), torch.float32, q.device)
    _check(lib().attn_full_decode(_dtype_code(q), B, H, d, scale, cap, max_pos, pp, *ptrs, kc, vc,
                                  op, lp, wp, workspace.numel() * workspace.element_size(),
                                  _stream()),
           "attn_full_decode")
    return o, lse


def attn_full_decode_noalloc(q, k_new, v_new, k_cache, v_cache, pos, max_pos: int, scale=None,
                             o=None, lse=None):
    """attn_full_decode with its split-KV partials in the library's fixed
    per-GPU scratch array: the C call allocates nothing (pass ``o`` and
    ``lse`` to allocate nothing here either).  Calls that overlap on one GPU
    share that array and race."""
    torch = _torch()
    B, H, d, o, lse, ptrs = _decode_io(q, k_new, v_new, o, lse)
    cap = k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kc = _dev(k_cache, "k_cache", (B, H, cap, d), q.dtype, q.device)
    vc = _dev(v_cache, "v_cache", (B, H, cap, d), q.dtype, q.device)
    pp = _dev(pos, "pos", (B,), torch.int64, q.device)
    op = _dev(o, "o", q.shape, q.dtype, q.device)
    lp = _dev(lse, "lse", (B, H), torch.float32, q.device)
    with torch.cuda.device(q.device):
        _check(lib().attn_full_decode_noalloc(_dtype_code(q), B, H, d, scale, cap, max_pos, pp, *ptrs,
                                              kc, vc, op, lp, _stream()),
               "attn_full_decode_noalloc")
    return o, lse


def attn_paged_decode(q, k_new, v_new, k_pages, v_pages, block_table, pos, max_pos: int,
                      scale=None, o=None, lse=None, workspace=None):
    """Decode one token per sequence against a paged full cache: pools
    [n_pages,H,64,d] and a block table [B,max_pages] int32."""
    torch = _torch()
    B, H, d, o, lse, ptrs = _decode_io(q, k_new, v_new, o, lse)
    n_pages = k_pages.shape[0]
    max_pages = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kp = _dev(k_pages, "k_pages", (n_pages, H, BLOCK, d), q.dtype, q.device)
    vp = _dev(v_pages, "v_pages", (n_pages, H, BLOCK, d), q.dtype, q.device)
    tp = _dev(block_table, "block_table", (B, max_pages), torch.int32, q.device)
    pp = _dev(pos, "pos", (B,), torch.int64, q.device)
    need = attn_workspace_bytes(ATTN_OP_FULL_DECODE, _dtype_code(q), B, H, max_pos + 1, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace", device=q.device)
    op = _dev(o, "o", q.shape, q.dtype, q.device)
    lp = _dev(lse, "lse", (B, H), torch.float32, q.device)
    _check(lib().attn_paged_decode(_dtype_code(q), B, H, d, scale, n_pages, max_pages, tp, max_pos,
                                   pp, *ptrs, kp, vp, op, lp, wp,
                                   workspace.numel() * workspace.element_size(), _stream()),
           "attn_paged_decode")
    return o, lse


def attn_paged_cache_fill(k_src, v_src, lengths, k_pages, v_pages, block_table):
    """Copies each sequence's prefill K/V [B,H,src_len,d] into its pages."""
    torch = _torch()
    B, H, src_len, d = k_src.shape
    n_pages = k_pages.shape[0]
    max_pages = block_table.shape[1]
    ks = _dev(k_src, "k_src", dtype=torch.bfloat16)
    vs = _dev(v_src, "v_src", k_src.shape, torch.bfloat16, k_src.device)
    lp = _dev(lengths, "lengths", (B,), torch.int64, k_src.device)
    kp = _dev(k_pages, "k_pages", (n_pages, H, BLOCK, d), torch.bfloat16, k_src.device)
    vp = _dev(v_pages, "v_pages", (n_pages, H, BLOCK, d), torch.bfloat16, k_src.device)
    tp = _dev(block_table, "block_table", (B, max_pages), torch.int32, k_src.device)
    _check(lib().attn_paged_cache_fill(ATTN_BF16, B, H, d, n_pages, max_pages, tp, lp, ks, vs,
                                       src_len, kp, vp, _stream()),
           "attn_paged_cache_fill")


def attn_ring_fill(k_src, v_src, lengths, k_cache, v_cache, sink_tokens: int, window_tokens: int):
    """Copies each sequence's sink and last-window tokens into a ring cache."""
    torch = _torch()
    B, H, src_len, d = k_src.shape
    S = sink_tokens + window_tokens
    ks = _dev(k_src, "k_src", dtype=torch.bfloat16)
    vs = _dev(v_src, "v_src", k_src.shape, torch.bfloat16, k_src.device)
    lp = _dev(lengths, "lengths", (B,), torch.int64, k_src.device)
    kc = _dev(k_cache, "k_cache", (B, H, S, d), torch.bfloat16, k_src.device)
    vc = _dev(v_cache, "v_cache", (B, H, S, d), torch.bfloat16, k_src.device)
    _check(lib().attn_ring_fill(ATTN_BF16, B, H, d, sink_tokens, window_tokens, lp, ks, vs,
                                src_len, kc, vc, _stream()), "attn_ring_fill")


def attn_blocksparse_cache_slots(pattern: Pattern, strided_blocks: int) -> int:
    """Slots per (b, h) of a BlockSparse compacted cache."""
    out = ctypes.c_int64(0)
    pat = pattern.c_struct()
    _check(lib().attn_blocksparse_cache_slots(ctypes.byref(pat), strided_blocks, ctypes.byref(out)),
           "attn_blocksparse_cache_slots")
    return out.value


def attn_blocksparse_strided_capacity(pattern: Pattern, max_tokens: int) -> int:
    """Strided-area blocks that positions below ``max_tokens`` can need (the
    largest count over the heads' stride phases)."""
    out = ctypes.c_int32(0)
    pat = pattern.c_struct()
    _check(lib().attn_blocksparse_strided_capacity(ctypes.byref(pat), max_tokens, ctypes.byref(out)),
           "attn_blocksparse_strided_capacity")
    return out.value


# shorter names used by callers
blocksparse_cache_slots = attn_blocksparse_cache_slots
blocksparse_strided_capacity = attn_blocksparse_strided_capacity


def attn_blocksparse_decode(q, k_new, v_new, k_cache, v_cache, pos, pattern: Pattern,
                            strided_blocks: int, scale=None, o=None, lse=None, workspace=None):
    """Decode one token per sequence of a BlockSparse layer against its
    compacted cache [B,H,64*(sink+local+strided_blocks),d]."""
    torch = _torch()
    B, H, d, o, lse, ptrs = _decode_io(q, k_new, v_new, o, lse)
    S = blocksparse_cache_slots(pattern, strided_blocks)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    kc = _dev(k_cache, "k_cache", (B, H, S, d), q.dtype, q.device)
    vc = _dev(v_cache, "v_cache", (B, H, S, d), q.dtype, q.device)
    pp = _dev(pos, "pos", (B,), torch.int64, q.device)
    need = attn_workspace_bytes(ATTN_OP_BLOCKSPARSE_DECODE, _dtype_code(q), B, H, S, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace", device=q.device)
    op = _dev(o, "o", q.shape, q.dtype, q.device)
    lp = _dev(lse, "lse", (B, H), torch.float32, q.device)
    pat = pattern.c_struct()
    _check(lib().attn_blocksparse_decode(_dtype_code(q), B, H, d, scale, ctypes.byref(pat),
                                         strided_blocks, pp, *ptrs, kc, vc, op, lp, wp,
                                         workspace.numel() * workspace.element_size(), _stream()),
           "attn_blocksparse_decode")
    return o, lse


def attn_blocksparse_cache_fill(k_src, v_src, lengths, k_cache, v_cache, pattern: Pattern,
                                strided_blocks: int):
    """Fills a BlockSparse compacted cache from prefill K/V."""
    torch = _torch()
    B, H, src_len, d = k_src.shape
    S = blocksparse_cache_slots(pattern, strided_blocks)
    ks = _dev(k_src, "k_src", dtype=torch.bfloat16)
    vs = _dev(v_src, "v_src", k_src.shape, torch.bfloat16, k_src.device)
    lp = _dev(lengths, "lengths", (B,), torch.int64, k_src.device)
    kc = _dev(k_cache, "k_cache", (B, H, S, d), torch.bfloat16, k_src.device)
    vc = _dev(v_cache, "v_cache", (B, H, S, d), torch.bfloat16, k_src.device)
    pat = pattern.c_struct()
    _check(lib().attn_blocksparse_cache_fill(ATTN_BF16, B, H, d, ctypes.byref(pat), strided_blocks,
                                             lp, ks, vs, src_len, kc, vc, _stream()),
           "attn_blocksparse_cache_fill")
