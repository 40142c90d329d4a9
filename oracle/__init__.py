"""TEST INFRASTRUCTURE ONLY: ctypes access to the double-precision CPU oracle
of the four-route SRNL forward pass (``srnl_oracle.c``).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package. The HIP library never does, and this package never
imports the library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "srnl_oracle.c")
LIB_PATH = os.path.join(_HERE, "libsrnl_oracle.so")
# The same source built with every state, product and sum in IEEE single
# precision. Not a reference: it measures how far an fp32 evaluation of the
# recurrence can drift from the double result on a given input (the
# conditioning of each chunk), which sets the per-chunk parity bar.
LIB32_PATH = os.path.join(_HERE, "libsrnl_oracle_f32.so")

CAP_SOFT, CAP_HARD, CAP_OFF = 0, 1, 2
TRACE_W = 18


def build() -> str:
    """Compile the oracle with plain gcc (IEEE double, no fast-math, no
    contraction of products into fused multiply-adds), and its fp32 build."""
    for path, extra in ((LIB_PATH, []), (LIB32_PATH, ["-DSRNL_ORACLE_REAL=float"])):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
               "-Wextra"] + extra + ["-o", path + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(path + ".tmp", path)
    return LIB_PATH


class _Opts(ctypes.Structure):
    _fields_ = [("alpha_max", ctypes.c_double), ("eps", ctypes.c_double),
                ("chunk_row", ctypes.c_int), ("chunk_col", ctypes.c_int),
                ("cap_mode", ctypes.c_int), ("clamp", ctypes.c_int),
                ("fixed_alpha", ctypes.c_int),
                ("readout_before", ctypes.c_int),
                ("freeze_kv", ctypes.c_int)]


_libs = {}


def lib(precision: str = "f64"):
    """The oracle library: "f64" (the reference) or "f32" (conditioning
    measurements only)."""
    if precision not in _libs:
        path = {"f64": LIB_PATH, "f32": LIB32_PATH}[precision]
        if any(not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(_SRC)
               for p in (LIB_PATH, LIB32_PATH)):
            build()
        L = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        L.srnl_oracle_scan.argtypes = [dp, dp] + [ctypes.c_int] * 6 + [
            ctypes.c_uint, dp, ctypes.POINTER(_Opts), dp, dp]
        L.srnl_oracle_scan.restype = ctypes.c_int
        L.srnl_oracle_fuse.argtypes = [dp] + [ctypes.c_int] * 4 + [
            ctypes.c_uint, dp, dp]
        L.srnl_oracle_fuse.restype = ctypes.c_int
        L.srnl_oracle_route_index.argtypes = [ctypes.c_int] * 3 + [
            ctypes.c_long, ctypes.POINTER(ctypes.c_int),
            ctypes.POINTER(ctypes.c_int)]
        L.srnl_oracle_route_index.restype = None
        L.srnl_oracle_chunk_len.argtypes = [ctypes.c_int] * 5
        L.srnl_oracle_chunk_len.restype = ctypes.c_int
        _libs[precision] = L
    return _libs[precision]


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def perturbed(a, k: int):
    """a (None allowed) with every element multiplied by 1 +- 2^-24, the fp32
    rounding unit, with signs drawn from numpy's seeded generator (seed
    1000 + k), in float64. The fp32 build run on such copies gives further
    fp32 evaluations of a problem that fp32 cannot tell from the original:
    their spread on a chunk measures that chunk's conditioning."""
    if a is None:
        return None
    rng = np.random.default_rng(1000 + k)
    return np.asarray(a, np.float64) * (1.0 + 2.0 ** -24 * rng.choice([-1.0, 1.0], np.shape(a)))


def route_index(r: int, H: int, W: int, t: int):
    i, j = ctypes.c_int(), ctypes.c_int()
    lib().srnl_oracle_route_index(r, H, W, t, ctypes.byref(i), ctypes.byref(j))
    return i.value, j.value


def chunk_len(r: int, H: int, W: int, chunk_row: int = 0, chunk_col: int = 0) -> int:
    return lib().srnl_oracle_chunk_len(r, H, W, chunk_row, chunk_col)


def scan(x, states, heads: int, d: int, route_mask: int = 15, q=None, *,
         alpha_max: float = 0.9, eps: float = 1e-6, chunk_row: int = 0,
         chunk_col: int = 0, cap_mode: int = CAP_SOFT, clamp: bool = True,
         fixed_alpha: bool = False, readout_before: bool = False,
         freeze_kv: bool = False, trace: bool = False, threads: int = 1,
         precision: str = "f64"):
    """Per-route outputs y [R][B][H*W][C] (traversal order) in float64.

    ``threads`` > 1 splits the batch over Python threads (each runs the
    single-threaded oracle on its own slice; ctypes releases the GIL).
    ``precision="f32"`` runs the fp32 build (conditioning measurements, not a
    reference). Returns y, or (y, trace) when ``trace`` is set."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, H, W, C = x.shape
    st = np.ascontiguousarray(states, dtype=np.float64)
    qq = None if q is None else np.ascontiguousarray(q, dtype=np.float64)
    R = bin(route_mask & 15).count("1")
    N = H * W
    opts = _Opts(alpha_max, eps, chunk_row, chunk_col, cap_mode, int(clamp),
                 int(fixed_alpha), int(readout_before), int(freeze_kv))

    def run(b0, b1):
        xs = np.ascontiguousarray(x[b0:b1])
        qs = None if qq is None else np.ascontiguousarray(qq[b0:b1])
        ys = np.zeros((R, b1 - b0, N, C))
        tr = np.zeros((R, b1 - b0, heads, N, TRACE_W)) if trace else None
        rc = lib(precision).srnl_oracle_scan(_p(xs), _p(qs), b1 - b0, H, W, C, heads, d,
                                    route_mask, _p(st), ctypes.byref(opts),
                                    _p(ys), _p(tr))
        if rc != 0:
            raise ValueError(f"srnl_oracle_scan returned {rc}")
        return ys, tr

    nt = max(1, min(threads, B))
    bounds = [(B * k // nt, B * (k + 1) // nt) for k in range(nt)]
    if nt == 1:
        parts = [run(0, B)]
    else:
        with ThreadPoolExecutor(nt) as ex:
            parts = list(ex.map(lambda ab: run(*ab), bounds))
    y = np.concatenate([p[0] for p in parts], axis=1)
    if trace:
        return y, np.concatenate([p[1] for p in parts], axis=1)
    return y


def scan_1d(x, states, heads: int, d: int, q=None, *, chunk: int = 0, **kw):
    """Standalone 1-D SRNL [README SRNL and VisionHOPE operator]: x [B][N][C]
    scanned once in token order, chunks of ``chunk`` tokens (0 selects the
    1-D default of 64; the last chunk may be short). The sequence is the
    row-major route of a 1 x N grid, so this is ``scan`` on that grid with
    route 0. ``states`` is [heads][3d^2+2d]. Returns y [B][N][C] in float64."""
    x = np.asarray(x)
    B, N, C = x.shape
    st = np.zeros((4,) + tuple(np.shape(states)), dtype=np.float64)
    st[0] = states
    qq = None if q is None else np.asarray(q).reshape(B, 1, N, C)
    y = scan(x.reshape(B, 1, N, C), st, heads, d, 1, qq,
             chunk_row=chunk if chunk > 0 else 64, **kw)
    return y[0]


def fuse(y, B: int, H: int, W: int, C: int, route_mask: int, scales):
    """Restored and fused output [B,H,W,C] in float64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    sc = np.ascontiguousarray(scales, dtype=np.float64)
    out = np.zeros((B, H, W, C))
    rc = lib().srnl_oracle_fuse(_p(y), B, H, W, C, route_mask, _p(sc), _p(out))
    if rc != 0:
        raise ValueError(f"srnl_oracle_fuse returned {rc}")
    return out


def forward(wl, route_mask: Optional[int] = None, threads: int = 1, **kw):
    """Scan + fuse of a synthetic workload (``synth.Workload``)."""
    rm = wl.route_mask if route_mask is None else route_mask
    y = scan(wl.x, wl.states, wl.heads, wl.d, rm, wl.q, alpha_max=wl.alpha_max,
             eps=wl.eps, chunk_row=wl.chunk_row, chunk_col=wl.chunk_col,
             threads=threads, **kw)
    return y, fuse(y, wl.B, wl.H, wl.W, wl.C, rm, wl.scales)
