"""Thin ctypes binding over libsrnl.so (C ABI in include/srnl.h).

Argument marshalling only: tensors are passed as device pointers with the
caller's current HIP stream; every step of the operator runs in the library's
kernels. The library must be built (``python -m
self_referential_memory_amd.build`` or ``__graft_entry__.build()``); loading
fails loudly when it is missing. There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsrnl.so")

SRNL_OK, SRNL_ERR_ARG, SRNL_ERR_DTYPE, SRNL_ERR_PTR, SRNL_ERR_WORKSPACE, SRNL_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
SRNL_ERR_NONFINITE = -6
SRNL_F32, SRNL_BF16 = 0, 1
FLAG_HARD_CAP, FLAG_NO_CAP, FLAG_NO_CLAMP, FLAG_FIXED_ALPHA, FLAG_READ_BEFORE = (
    0x1, 0x2, 0x4, 0x8, 0x10)
FLAG_FREEZE_KV = 0x20
FLAG_CHECK_FINITE = 0x40
FLAG_RECORD = 0x80

EXPORTS = ("srnl_scan_fwd", "srnl_scan_workspace_bytes", "srnl_scan_1d",
           "srnl_scan_1d_workspace_bytes", "srnl_fuse", "srnl_scan_bwd",
           "srnl_scan_bwd_workspace_bytes", "srnl_scan_1d_bwd", "srnl_scan_1d_bwd_workspace_bytes",
           "srnl_fuse_bwd", "srnl_fuse_bwd_workspace_bytes", "srnl_fuse_bwd_noalloc",
           "srnl_scan_fuse_bwd", "srnl_scan_fuse_bwd_workspace_bytes",
           "srnl_route_gather", "srnl_init_states", "srnl_block_fwd",
           "srnl_block_workspace_bytes",
           "srnl_route_index", "srnl_chunk_len", "srnl_status_string",
           "srnl_last_error")


class SrnlError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("states", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("in_dtype", ctypes.c_int), ("alpha_max", ctypes.c_float),
                ("eps", ctypes.c_float), ("chunk_row", ctypes.c_int),
                ("chunk_col", ctypes.c_int), ("flags", ctypes.c_uint),
                ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class BlockWeights(ctypes.Structure):
    """srnl_block_weights: device pointers of the block parameters."""
    _fields_ = [("ln1_w", ctypes.c_void_p), ("ln1_b", ctypes.c_void_p),
                ("wq", ctypes.c_void_p), ("dw_w", ctypes.c_void_p), ("dw_b", ctypes.c_void_p),
                ("ln2_w", ctypes.c_void_p), ("ln2_b", ctypes.c_void_p),
                ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("ffn_hidden", ctypes.c_int),
                ("ln_eps", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsrnl.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
        L.srnl_scan_fwd.argtypes = [vp, i, i, i, i, i, i, u, ctypes.POINTER(Params), vp]
        L.srnl_scan_1d.argtypes = [vp, i, i, i, i, i, ctypes.POINTER(Params), vp]
        L.srnl_fuse.argtypes = [vp, i, i, i, i, u, vp, i, vp, vp]
        sz = ctypes.c_size_t
        L.srnl_scan_workspace_bytes.argtypes = [i, i, i, i, i, i, u, ctypes.POINTER(Params)]
        L.srnl_scan_workspace_bytes.restype = sz
        L.srnl_scan_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, u, ctypes.POINTER(Params)]
        L.srnl_scan_bwd_workspace_bytes.restype = sz
        L.srnl_scan_bwd.argtypes = [vp, i, i, i, i, i, i, u, ctypes.POINTER(Params), vp, vp, sz,
                                    vp, vp, vp]
        L.srnl_scan_1d_workspace_bytes.argtypes = [i, i, i, i, i, ctypes.POINTER(Params)]
        L.srnl_scan_1d_workspace_bytes.restype = sz
        L.srnl_scan_1d_bwd_workspace_bytes.argtypes = [i, i, i, i, i, ctypes.POINTER(Params)]
        L.srnl_scan_1d_bwd_workspace_bytes.restype = sz
        L.srnl_scan_1d_bwd.argtypes = [vp, i, i, i, i, i, ctypes.POINTER(Params), vp, vp, sz,
                                       vp, vp, vp]
        L.srnl_fuse_bwd_workspace_bytes.argtypes = [i, i, i, i, u]
        L.srnl_fuse_bwd_workspace_bytes.restype = sz
        L.srnl_fuse_bwd.argtypes = [vp, vp, i, i, i, i, u, vp, vp, vp, vp, sz, vp]
        L.srnl_fuse_bwd_noalloc.argtypes = [vp, vp, i, i, i, i, u, vp, vp, vp, vp]
        L.srnl_scan_fuse_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, u, ctypes.POINTER(Params)]
        L.srnl_scan_fuse_bwd_workspace_bytes.restype = sz
        L.srnl_scan_fuse_bwd.argtypes = [vp, i, i, i, i, i, i, u, ctypes.POINTER(Params), vp, vp,
                                         vp, vp, sz, vp, vp, vp, vp]
        L.srnl_route_gather.argtypes = [vp, i, i, i, i, u, i, vp, vp]
        L.srnl_init_states.argtypes = [vp, i, i, ctypes.c_ulonglong, ctypes.c_float, vp]
        L.srnl_block_workspace_bytes.argtypes = [i, i, i, i, u]
        L.srnl_block_workspace_bytes.restype = sz
        L.srnl_block_fwd.argtypes = [vp, i, i, i, i, i, i, u, ctypes.POINTER(Params),
                                     ctypes.POINTER(BlockWeights), vp, sz, vp]
        for f in ("srnl_scan_fwd", "srnl_scan_1d", "srnl_fuse", "srnl_scan_bwd",
                  "srnl_scan_1d_bwd", "srnl_fuse_bwd", "srnl_fuse_bwd_noalloc",
                  "srnl_scan_fuse_bwd", "srnl_route_gather", "srnl_init_states", "srnl_block_fwd"):
            getattr(L, f).restype = ctypes.c_int
        L.srnl_route_index.argtypes = [i, i, i, ctypes.c_long, ctypes.POINTER(i),
                                       ctypes.POINTER(i)]
        L.srnl_route_index.restype = None
        L.srnl_chunk_len.argtypes = [i, i, i, i, i]
        L.srnl_chunk_len.restype = ctypes.c_int
        L.srnl_status_string.argtypes = [i]
        L.srnl_status_string.restype = ctypes.c_char_p
        L.srnl_last_error.argtypes = []
        L.srnl_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != SRNL_OK:
        raise SrnlError(status, where, lib().srnl_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], shape, dtype, name: str) -> None:
    """The library sees only pointers: buffer shapes and dtypes are checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _state_shape(heads: int, d: int):
    return (4, heads, 3 * d * d + 2 * d)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _keep_for_stream(handle, *tensors) -> None:
    """Temporaries this binding allocates (on the current stream) and frees
    on return, but whose kernels run on the stream ``handle``: record that
    stream on them, so the caching allocator does not hand their memory out
    again before that stream's work is done."""
    cur = torch.cuda.current_stream()
    if (handle or 0) == (cur.cuda_stream or 0):
        return
    s = torch.cuda.ExternalStream(handle) if handle else torch.cuda.default_stream()
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SRNL_F32
    if t.dtype == torch.bfloat16:
        return SRNL_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def route_index(r: int, H: int, W: int, t: int):
    i, j = ctypes.c_int(), ctypes.c_int()
    lib().srnl_route_index(r, H, W, t, ctypes.byref(i), ctypes.byref(j))
    return i.value, j.value


def chunk_len(r: int, H: int, W: int, chunk_row: int = 0, chunk_col: int = 0) -> int:
    return lib().srnl_chunk_len(r, H, W, chunk_row, chunk_col)


def make_params(states: torch.Tensor, x: torch.Tensor, q: Optional[torch.Tensor] = None, *,
                alpha_max: float = 0.9, eps: float = 1e-6, chunk_row: int = 0,
                chunk_col: int = 0, flags: int = 0, stream=None) -> Params:
    if q is not None and (q.dtype != x.dtype or q.shape != x.shape):
        raise SrnlError(SRNL_ERR_DTYPE, "make_params",
                        "separate queries must have the shape and dtype of x")
    return Params(_ptr(states), _ptr(q), _dtype_code(x), alpha_max, eps, chunk_row,
                  chunk_col, flags, _stream(stream))


def _finite_check_workspace(p: Params, x: torch.Tensor, nbytes: int):
    """With SRNL_FLAG_CHECK_FINITE and no caller workspace, allocate one of
    nbytes (the entry point's workspace query) and point p at it; the call
    waits for its stream when checking, so the buffer outlives its use.
    Returns the tensor (None when nothing was allocated). A record
    (SRNL_FLAG_RECORD) must outlive the call: that takes scan_fwd_record
    (scan_1d_record) or a caller workspace."""
    if p.workspace or not nbytes:
        return None
    if p.flags & FLAG_RECORD and nbytes > (256 if p.flags & FLAG_CHECK_FINITE else 0):
        raise ValueError("FLAG_RECORD needs a workspace that outlives the call: use "
                         "scan_fwd_record (scan_1d_record), which returns the record, or "
                         "pass params with a workspace")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    p.workspace, p.workspace_bytes = ws.data_ptr(), nbytes
    return ws


def scan_fwd(x: torch.Tensor, states: torch.Tensor, heads: int, d: int,
             route_mask: int = 15, q: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, *, params: Optional[Params] = None,
             **kw) -> torch.Tensor:
    """srnl_scan_fwd: x [B,H,W,C] -> per-route outputs [R,B,H*W,C] fp32."""
    B, H, W, C = x.shape
    R = bin(route_mask & 15).count("1")
    _expect(states, _state_shape(heads, d), torch.float32, "states")
    if out is None:
        out = torch.empty((R, B, H * W, C), dtype=torch.float32, device=x.device)
    _expect(out, (R, B, H * W, C), torch.float32, "out")
    p = params if params is not None else make_params(states, x, q, **kw)
    nbytes = 0 if p.workspace else lib().srnl_scan_workspace_bytes(
        B, H, W, C, heads, d, route_mask, ctypes.byref(p))
    ws = _finite_check_workspace(p, x, nbytes)
    try:
        _check(lib().srnl_scan_fwd(_ptr(x), B, H, W, C, heads, d, route_mask,
                                   ctypes.byref(p), _ptr(out)), "srnl_scan_fwd")
    finally:
        if ws is not None:
            p.workspace, p.workspace_bytes = None, 0
    return out


def scan_fwd_record(x: torch.Tensor, states: torch.Tensor, heads: int, d: int,
                    route_mask: int = 15, q: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, *, flags: int = 0, **kw):
    """srnl_scan_fwd with SRNL_FLAG_RECORD: the route outputs [R,B,H*W,C] and
    the forward record (a uint8 device tensor, or None where the windowed
    backward does not apply) for scan_bwd(..., record=...)."""
    B, H, W, C = x.shape
    R = bin(route_mask & 15).count("1")
    _expect(states, _state_shape(heads, d), torch.float32, "states")
    if out is None:
        out = torch.empty((R, B, H * W, C), dtype=torch.float32, device=x.device)
    _expect(out, (R, B, H * W, C), torch.float32, "out")
    p = make_params(states, x, q, flags=flags | FLAG_RECORD, **kw)
    only = Params.from_buffer_copy(p)
    only.flags &= ~FLAG_CHECK_FINITE
    rec_bytes = lib().srnl_scan_workspace_bytes(B, H, W, C, heads, d, route_mask,
                                                ctypes.byref(only))
    nbytes = lib().srnl_scan_workspace_bytes(B, H, W, C, heads, d, route_mask, ctypes.byref(p))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    if ws is not None:
        p.workspace, p.workspace_bytes = ws.data_ptr(), nbytes
    _check(lib().srnl_scan_fwd(_ptr(x), B, H, W, C, heads, d, route_mask, ctypes.byref(p),
                               _ptr(out)), "srnl_scan_fwd")
    rec = ws[:rec_bytes] if rec_bytes else None
    return out, rec


def scan_1d(x: torch.Tensor, states: torch.Tensor, heads: int, d: int,
            q: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, *,
            chunk: int = 0, params: Optional[Params] = None, **kw) -> torch.Tensor:
    """srnl_scan_1d: x [B,N,C] -> y [B,N,C] fp32 (chunk 0 selects 64 tokens)."""
    B, N, C = x.shape
    _expect(states, (heads, 3 * d * d + 2 * d), torch.float32, "states")
    if out is None:
        out = torch.empty((B, N, C), dtype=torch.float32, device=x.device)
    _expect(out, (B, N, C), torch.float32, "out")
    p = params if params is not None else make_params(states, x, q, chunk_row=chunk, **kw)
    nbytes = 0 if p.workspace else lib().srnl_scan_1d_workspace_bytes(
        B, N, C, heads, d, ctypes.byref(p))
    ws = _finite_check_workspace(p, x, nbytes)
    try:
        _check(lib().srnl_scan_1d(_ptr(x), B, N, C, heads, d, ctypes.byref(p), _ptr(out)),
               "srnl_scan_1d")
    finally:
        if ws is not None:
            p.workspace, p.workspace_bytes = None, 0
    return out


def scan_1d_record(x: torch.Tensor, states: torch.Tensor, heads: int, d: int,
                   q: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, *,
                   chunk: int = 0, flags: int = 0, **kw):
    """srnl_scan_1d with SRNL_FLAG_RECORD: y [B,N,C] and the forward record
    (a uint8 device tensor, or None where the windowed backward does not
    apply) for scan_1d_bwd(..., record=...)."""
    B, N, C = x.shape
    _expect(states, (heads, 3 * d * d + 2 * d), torch.float32, "states")
    if out is None:
        out = torch.empty((B, N, C), dtype=torch.float32, device=x.device)
    _expect(out, (B, N, C), torch.float32, "out")
    p = make_params(states, x, q, chunk_row=chunk, flags=flags | FLAG_RECORD, **kw)
    only = Params.from_buffer_copy(p)
    only.flags &= ~FLAG_CHECK_FINITE
    rec_bytes = lib().srnl_scan_1d_workspace_bytes(B, N, C, heads, d, ctypes.byref(only))
    nbytes = lib().srnl_scan_1d_workspace_bytes(B, N, C, heads, d, ctypes.byref(p))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    if ws is not None:
        p.workspace, p.workspace_bytes = ws.data_ptr(), nbytes
    _check(lib().srnl_scan_1d(_ptr(x), B, N, C, heads, d, ctypes.byref(p), _ptr(out)),
           "srnl_scan_1d")
    return out, (ws[:rec_bytes] if rec_bytes else None)


def scan_1d_bwd(x: torch.Tensor, states: torch.Tensor, heads: int, d: int, dy: torch.Tensor,
                q: Optional[torch.Tensor] = None, *, chunk: int = 0,
                record: Optional[torch.Tensor] = None, **kw):
    """srnl_scan_1d_bwd: dy [B,N,C] fp32 -> (dx [B,N,C], dq or None, dstates
    [heads,3d^2+2d]), all fp32, for srnl_scan_1d's forward with the same
    arguments (chunk 0 selects 64 tokens). ``record``: the forward record
    from scan_1d_record. The workspace is allocated here (torch)."""
    B, N, C = x.shape
    _expect(states, (heads, 3 * d * d + 2 * d), torch.float32, "states")
    _expect(dy, (B, N, C), torch.float32, "dy")
    p = make_params(states, x, q, chunk_row=chunk, **kw)
    if record is not None:
        p.flags = (p.flags | FLAG_RECORD) & ~FLAG_CHECK_FINITE
        p.workspace, p.workspace_bytes = record.data_ptr(), record.numel() * record.element_size()
    nbytes = lib().srnl_scan_1d_bwd_workspace_bytes(B, N, C, heads, d, ctypes.byref(p))
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x.device)
    dx = torch.empty((B, N, C), dtype=torch.float32, device=x.device)
    dq = None if q is None else torch.empty_like(dx)
    dst = torch.empty((heads, 3 * d * d + 2 * d), dtype=torch.float32, device=x.device)
    _check(lib().srnl_scan_1d_bwd(_ptr(x), B, N, C, heads, d, ctypes.byref(p), _ptr(dy),
                                  _ptr(ws), int(nbytes), _ptr(dx), _ptr(dq), _ptr(dst)),
           "srnl_scan_1d_bwd")
    _keep_for_stream(p.stream, ws)
    return dx, dq, dst


def fuse(y: torch.Tensor, B: int, H: int, W: int, C: int, route_mask: int,
         scales: torch.Tensor, out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
         stream=None) -> torch.Tensor:
    """srnl_fuse: per-route outputs -> restored, channel-scaled sum [B,H,W,C]."""
    R = bin(route_mask & 15).count("1")
    _expect(y, (R, B, H * W, C), torch.float32, "y")
    _expect(scales, (4, C), torch.float32, "scales")
    if out is None:
        out = torch.empty((B, H, W, C), dtype=out_dtype, device=y.device)
    _check(lib().srnl_fuse(_ptr(y), B, H, W, C, route_mask, _ptr(scales),
                           _dtype_code(out), _ptr(out), _stream(stream)), "srnl_fuse")
    return out


def scan_bwd(x: torch.Tensor, states: torch.Tensor, heads: int, d: int, dy: torch.Tensor,
             route_mask: int = 15, q: Optional[torch.Tensor] = None, *,
             params: Optional[Params] = None, record: Optional[torch.Tensor] = None, **kw):
    """srnl_scan_bwd: dy [R,B,H*W,C] fp32 -> (dx [B,H,W,C], dq or None, dstates
    [4,heads,3d^2+2d]), all fp32. The workspace is allocated here (torch).
    ``record``: the forward record from scan_fwd_record with the same
    arguments; the backward then reads it instead of recomputing it."""
    B, H, W, C = x.shape
    R = bin(route_mask & 15).count("1")
    _expect(states, _state_shape(heads, d), torch.float32, "states")
    _expect(dy, (R, B, H * W, C), torch.float32, "dy")
    p = params if params is not None else make_params(states, x, q, **kw)
    if record is not None:
        p = Params.from_buffer_copy(p)
        p.flags = (p.flags | FLAG_RECORD) & ~FLAG_CHECK_FINITE
        p.workspace, p.workspace_bytes = record.data_ptr(), record.numel() * record.element_size()
    nbytes = lib().srnl_scan_bwd_workspace_bytes(B, H, W, C, heads, d, route_mask, ctypes.byref(p))
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x.device)
    dx = torch.empty((B, H, W, C), dtype=torch.float32, device=x.device)
    dq = None if q is None else torch.empty_like(dx)
    dst = torch.empty((4, heads, 3 * d * d + 2 * d), dtype=torch.float32, device=x.device)
    _check(lib().srnl_scan_bwd(_ptr(x), B, H, W, C, heads, d, route_mask, ctypes.byref(p),
                               _ptr(dy), _ptr(ws), int(nbytes), _ptr(dx), _ptr(dq), _ptr(dst)),
           "srnl_scan_bwd")
    _keep_for_stream(p.stream, ws)
    return dx, dq, dst


def fuse_bwd(dout: torch.Tensor, y: torch.Tensor, B: int, H: int, W: int, C: int,
             route_mask: int, scales: torch.Tensor, stream=None):
    """srnl_fuse_bwd: dout [B,H,W,C] fp32 -> (dy_routes [R,B,H*W,C], dscales [4,C])."""
    R = bin(route_mask & 15).count("1")
    _expect(dout, (B, H, W, C), torch.float32, "dout")
    _expect(y, (R, B, H * W, C), torch.float32, "y")
    _expect(scales, (4, C), torch.float32, "scales")
    nbytes = lib().srnl_fuse_bwd_workspace_bytes(B, H, W, C, route_mask)
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dout.device)
    dyr = torch.empty_like(y)
    dsc = torch.empty((4, C), dtype=torch.float32, device=dout.device)
    sh = _stream(stream)
    _check(lib().srnl_fuse_bwd(_ptr(dout), _ptr(y), B, H, W, C, route_mask, _ptr(scales),
                               _ptr(dyr), _ptr(dsc), _ptr(ws), int(nbytes), sh),
           "srnl_fuse_bwd")
    _keep_for_stream(sh, ws)
    return dyr, dsc


def scan_fuse_bwd(x: torch.Tensor, states: torch.Tensor, heads: int, d: int, y: torch.Tensor,
                  scales: torch.Tensor, dout: torch.Tensor, route_mask: int = 15,
                  q: Optional[torch.Tensor] = None, *, params: Optional[Params] = None,
                  record: Optional[torch.Tensor] = None, **kw):
    """srnl_scan_fuse_bwd: the operator's backward in one call, dout [B,H,W,C]
    fp32 -> (dx [B,H,W,C], dq or None, dstates [4,heads,3d^2+2d], dscales
    [4,C]), all fp32; the same results as fuse_bwd then scan_bwd. y: the
    forward's route outputs [R,B,H*W,C]; ``record`` as for scan_bwd."""
    B, H, W, C = x.shape
    R = bin(route_mask & 15).count("1")
    _expect(states, _state_shape(heads, d), torch.float32, "states")
    _expect(y, (R, B, H * W, C), torch.float32, "y")
    _expect(scales, (4, C), torch.float32, "scales")
    _expect(dout, (B, H, W, C), torch.float32, "dout")
    p = params if params is not None else make_params(states, x, q, **kw)
    if record is not None:
        p = Params.from_buffer_copy(p)
        p.flags = (p.flags | FLAG_RECORD) & ~FLAG_CHECK_FINITE
        p.workspace, p.workspace_bytes = record.data_ptr(), record.numel() * record.element_size()
    nbytes = lib().srnl_scan_fuse_bwd_workspace_bytes(B, H, W, C, heads, d, route_mask,
                                                      ctypes.byref(p))
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x.device)
    dx = torch.empty((B, H, W, C), dtype=torch.float32, device=x.device)
    dq = None if q is None else torch.empty_like(dx)
    dst = torch.empty((4, heads, 3 * d * d + 2 * d), dtype=torch.float32, device=x.device)
    dsc = torch.empty((4, C), dtype=torch.float32, device=x.device)
    _check(lib().srnl_scan_fuse_bwd(_ptr(x), B, H, W, C, heads, d, route_mask, ctypes.byref(p),
                                    _ptr(y), _ptr(scales), _ptr(dout), _ptr(ws), int(nbytes),
                                    _ptr(dx), _ptr(dq), _ptr(dst), _ptr(dsc)),
           "srnl_scan_fuse_bwd")
    _keep_for_stream(p.stream, ws)
    return dx, dq, dst, dsc


def route_gather(x: torch.Tensor, route_mask: int = 15, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """srnl_route_gather: x [B,H,W,C] -> [R,B,H*W,C] in route order."""
    B, H, W, C = x.shape
    R = bin(route_mask & 15).count("1")
    if out is None:
        out = torch.empty((R, B, H * W, C), dtype=x.dtype, device=x.device)
    _check(lib().srnl_route_gather(_ptr(x), B, H, W, C, route_mask, _dtype_code(x),
                                   _ptr(out), _stream(stream)), "srnl_route_gather")
    return out


def init_states(heads: int, d: int, seed: int, std: float, device="cuda",
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """srnl_init_states: [4, heads, 3d^2+2d] fp32 ~ std * N(0,1) (Philox)."""
    if out is None:
        out = torch.empty((4, heads, 3 * d * d + 2 * d), dtype=torch.float32, device=device)
    _check(lib().srnl_init_states(_ptr(out), heads, d, seed, std, _stream(stream)),
           "srnl_init_states")
    return out


def forward(x: torch.Tensor, states: torch.Tensor, scales: torch.Tensor, heads: int, d: int,
            route_mask: int = 15, q: Optional[torch.Tensor] = None, out_dtype=None,
            **kw) -> torch.Tensor:
    """Scan + fuse: the operator's forward pass on an NHWC grid."""
    B, H, W, C = x.shape
    y = scan_fwd(x, states, heads, d, route_mask, q, **kw)
    return fuse(y, B, H, W, C, route_mask, scales,
                out_dtype=x.dtype if out_dtype is None else out_dtype,
                stream=kw.get("stream"))


def _side_stream(kw):
    """The stream kw asks for when it is not the current one, else None."""
    s = kw.get("stream")
    if s is None:
        return None
    cur = torch.cuda.current_stream()
    return None if (s.cuda_stream or 0) == (cur.cuda_stream or 0) else s


class Operator(torch.autograd.Function):
    """The operator (scan + fuse) as an autograd node: the forward pass is
    srnl_scan_fwd and srnl_fuse, the backward pass srnl_scan_fuse_bwd (the
    results of srnl_fuse_bwd then srnl_scan_bwd). Gradients flow to x, the initial states, the scales and
    the separate queries. The route outputs are kept for the fusion backward,
    and, where the windowed backward applies, the forward's record
    (SRNL_FLAG_RECORD), so the backward does not run the forward again.

    With stream= (kw) another than the current stream, both passes run on
    that stream: it first waits for the current stream (the inputs, or the
    incoming gradient, are made there), everything the pass allocates is
    allocated on it, and the current stream then waits for it before the
    result is handed back; the results are recorded as used on the current
    stream, so the caching allocator keeps them until that stream is done."""

    @staticmethod
    def forward(ctx, x, states, scales, q, heads, d, route_mask, kw):
        B, H, W, C = x.shape
        side = _side_stream(kw)
        kwc = {k: v for k, v in kw.items() if k != "stream"}
        cur = torch.cuda.current_stream()
        if side is not None:
            side.wait_stream(cur)
        with torch.cuda.stream(side if side is not None else cur):
            y, rec = scan_fwd_record(x, states, heads, d, route_mask, q, **kwc)
            out = fuse(y, B, H, W, C, route_mask, scales, out_dtype=x.dtype)
        if side is not None:
            cur.wait_stream(side)
            out.record_stream(cur)
        ctx.save_for_backward(x, states, scales, q, y, rec)
        ctx.cfg = (heads, d, route_mask, kw)
        return out

    @staticmethod
    def backward(ctx, dout):
        x, states, scales, q, y, rec = ctx.saved_tensors
        heads, d, route_mask, kw = ctx.cfg
        B, H, W, C = x.shape
        side = _side_stream(kw)
        kwc = {k: v for k, v in kw.items() if k != "stream"}
        cur = torch.cuda.current_stream()
        if side is not None:
            side.wait_stream(cur)
            dout.record_stream(side)
        with torch.cuda.stream(side if side is not None else cur):
            d32 = dout.to(torch.float32).contiguous()
            dx, dq, dst, dsc = scan_fuse_bwd(x, states, heads, d, y, scales, d32, route_mask, q,
                                             record=rec, **kwc)
            grads = (dx.to(x.dtype), dst, dsc, None if dq is None else dq.to(q.dtype))
        if side is not None:
            cur.wait_stream(side)
            for g in grads:
                if g is not None:
                    g.record_stream(cur)
        return grads + (None, None, None, None)


def operator(x: torch.Tensor, states: torch.Tensor, scales: torch.Tensor, heads: int, d: int,
             route_mask: int = 15, q: Optional[torch.Tensor] = None, **kw) -> torch.Tensor:
    """Differentiable scan + fuse on an NHWC grid; the output has x's dtype.
    ``kw`` are the srnl_params fields (alpha_max, eps, chunk_row, chunk_col,
    flags)."""
    return Operator.apply(x, states, scales, q, heads, d, route_mask, kw)


def block_weights(bw: dict, scales: torch.Tensor, ln_eps: float = 1e-5) -> BlockWeights:
    """srnl_block_weights from a dict of device tensors: ln1_w, ln1_b, dw_w
    [C,3,3], dw_b, ln2_w, ln2_b, b1, b2 (fp32) and wq [C,C], w1 [F,C], w2
    [C,F] (bf16). The tensors must outlive the calls that use the struct."""
    # the library sees only pointers: every shape is checked here
    C = int(bw["wq"].shape[0])
    F = int(bw["w1"].shape[0])
    shapes = {"ln1_w": (C,), "ln1_b": (C,), "wq": (C, C), "dw_w": (C, 3, 3), "dw_b": (C,),
              "ln2_w": (C,), "ln2_b": (C,), "w1": (F, C), "b1": (F,), "w2": (C, F), "b2": (C,)}
    for k, shp in shapes.items():
        if tuple(bw[k].shape) != shp:
            raise ValueError(f"{k} has shape {tuple(bw[k].shape)}, expected {shp}")
        want = torch.bfloat16 if k in ("wq", "w1", "w2") else torch.float32
        if bw[k].dtype != want:
            raise ValueError(f"{k} must be {want}")
    if tuple(scales.shape) != (4, C) or scales.dtype != torch.float32:
        raise ValueError(f"scales must be float32 of shape (4, {C})")
    w = BlockWeights(_ptr(bw["ln1_w"]), _ptr(bw["ln1_b"]), _ptr(bw["wq"]), _ptr(bw["dw_w"]),
                     _ptr(bw["dw_b"]), _ptr(bw["ln2_w"]), _ptr(bw["ln2_b"]), _ptr(bw["w1"]),
                     _ptr(bw["b1"]), _ptr(bw["w2"]), _ptr(bw["b2"]), _ptr(scales), F, ln_eps)
    w.channels = C
    return w


def block_fwd(x: torch.Tensor, states: torch.Tensor, weights: BlockWeights, heads: int, d: int,
              route_mask: int = 15, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, *, params: Optional[Params] = None,
              **kw) -> torch.Tensor:
    """srnl_block_fwd: one residual block, x [B,H,W,C] -> out [B,H,W,C] in
    x's dtype. The workspace is allocated here (torch) unless given."""
    B, H, W, C = x.shape
    if getattr(weights, "channels", C) != C:
        raise ValueError(f"weights are for C = {weights.channels}, x has C = {C}")
    _expect(states, _state_shape(heads, d), torch.float32, "states")
    if out is None:
        out = torch.empty_like(x)
    _expect(out, x.shape, x.dtype, "out")
    nbytes = lib().srnl_block_workspace_bytes(B, H, W, C, route_mask)
    if workspace is not None and workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace smaller than srnl_block_workspace_bytes")
    own = workspace is None
    if own:
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x.device)
    p = params if params is not None else make_params(states, x, **kw)
    _check(lib().srnl_block_fwd(_ptr(x), B, H, W, C, heads, d, route_mask, ctypes.byref(p),
                                ctypes.byref(weights), _ptr(workspace),
                                int(workspace.numel() * workspace.element_size()),
                                _ptr(out)), "srnl_block_fwd")
    if own:
        _keep_for_stream(p.stream, workspace)
    return out
