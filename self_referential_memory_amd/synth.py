"""Seeded synthetic inputs for the four-route SRNL forward pass.

This module is shared by the tests, the benchmark and the oracle harness. It
draws random numbers and arranges them into the tensors the operator takes; it
holds none of the operator's arithmetic.

Random numbers come from Philox4x32-10, the counter-based generator published
by Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3",
SC'11), implemented here from that definition with numpy integer arithmetic.
Normals use the Box-Muller transform in double precision. Each tensor draws
from its own stream id, so the draw order between tensors does not matter:

  block k of stream s under seed S is Philox4x32-10 applied to the counter
  (k mod 2^32, k div 2^32, s, 0x53524E4C) with key (S mod 2^32, S div 2^32);
  it yields 4 uint32 words a0..a3; u(a) = (a + 0.5) * 2^-32 lies in (0, 1);
  normals 4k..4k+3 are r0 cos t0, r0 sin t0, r1 cos t1, r1 sin t1 with
  r0 = sqrt(-2 ln u(a0)), t0 = 2 pi u(a1), r1 = sqrt(-2 ln u(a2)), t1 = 2 pi u(a3).

The device-side state initialiser of the library (``srnl_init_states``)
implements the same generator for the STATES stream, so its output can be
checked against :func:`states` bit for bit (up to the last-ulp behaviour of the
two libms).

Workloads follow the grids the pages describe: the hierarchical backbone's
stage maps (224/4 ... 224/32), the plain backbone's 14x14 map and a dense
prediction map (800x1216 input / 4 = 200x304). They stand in for ImageNet/COCO
feature maps; no dataset item is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# Philox4x32 constants (Salmon et al. 2011, Table/Section on Philox).
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_TAG = 0x53524E4C  # "SRNL"
_MASK32 = np.uint64(0xFFFFFFFF)

STREAM_X = 1
STREAM_STATES = 2
STREAM_SCALES = 3
STREAM_OUTLIERS = 4
STREAM_Q = 5
STREAM_BLOCK = 6


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on uint32 arrays c0..c3 and a 2-word key."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + _PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + _PHILOX_W1) & 0xFFFFFFFF
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def raw_words(seed: int, stream: int, n: int) -> np.ndarray:
    """The first n uint32 words of a stream (4 per Philox block, in order)."""
    nb = (n + 3) // 4
    k = np.arange(nb, dtype=np.uint64)
    lo = (k & _MASK32).astype(np.uint32)
    hi = (k >> np.uint64(32)).astype(np.uint32)
    s = np.full(nb, stream, dtype=np.uint32)
    tag = np.full(nb, _TAG, dtype=np.uint32)
    a0, a1, a2, a3 = philox4x32_10(lo, hi, s, tag, seed & 0xFFFFFFFF,
                                   (seed >> 32) & 0xFFFFFFFF)
    return np.stack([a0, a1, a2, a3], axis=1).reshape(-1)[:n]


def uniforms(seed: int, stream: int, n: int) -> np.ndarray:
    """n doubles in (0, 1): u(a) = (a + 0.5) * 2^-32."""
    a = raw_words(seed, stream, n).astype(np.float64)
    return (a + 0.5) * (2.0 ** -32)


def normals(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normals (double) by Box-Muller over Philox words."""
    nb = (n + 3) // 4
    u = uniforms(seed, stream, 4 * nb).reshape(nb, 4)
    r0 = np.sqrt(-2.0 * np.log(u[:, 0]))
    t0 = 2.0 * math.pi * u[:, 1]
    r1 = np.sqrt(-2.0 * np.log(u[:, 2]))
    t1 = 2.0 * math.pi * u[:, 3]
    z = np.stack([r0 * np.cos(t0), r0 * np.sin(t0),
                  r1 * np.cos(t1), r1 * np.sin(t1)], axis=1)
    return z.reshape(-1)[:n]


def state_size(d: int) -> int:
    """Floats per (route, head): M_c, M_k, M_v (d x d each), m_eta, m_alpha."""
    return 3 * d * d + 2 * d


def states(seed: int, heads: int, d: int, std: float) -> np.ndarray:
    """Initial memories [4][heads][3d^2+2d] fp32, each entry std * N(0,1).
    std is taken at fp32 precision and the product formed in double, then
    rounded to fp32, as the library's state initialiser does."""
    n = 4 * heads * state_size(d)
    z = normals(seed, STREAM_STATES, n)
    s = np.float64(np.float32(std))
    return (s * z).astype(np.float32).reshape(4, heads, state_size(d))


def scales(seed: int, C: int, lo: float = 0.5, hi: float = 1.5) -> np.ndarray:
    """Channel fusion scales [4][C] fp32 ~ U(lo, hi)."""
    u = uniforms(seed, STREAM_SCALES, 4 * C)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(4, C)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the bf16
    values as fp32 and the raw uint16 words."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    words = r.astype(np.uint16)
    vals = (words.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, words


@dataclasses.dataclass
class BlockWeights:
    """Parameters of one residual block around the operator: layer norms,
    the shared query projection, the 3x3 depthwise convolution and the
    feed-forward network. The three projection matrices are bf16 values
    (kept as fp32 arrays that are exactly representable in bf16); everything
    else is fp32."""
    ln1_w: np.ndarray   # [C]
    ln1_b: np.ndarray   # [C]
    wq: np.ndarray      # [C][C]  q = u wq^T
    dw_w: np.ndarray    # [C][3][3]
    dw_b: np.ndarray    # [C]
    ln2_w: np.ndarray   # [C]
    ln2_b: np.ndarray   # [C]
    w1: np.ndarray      # [F][C]
    b1: np.ndarray      # [F]
    w2: np.ndarray      # [C][F]
    b2: np.ndarray      # [C]
    ln_eps: float = 1e-5

    @property
    def F(self) -> int:
        return self.w1.shape[0]


def block_weights(seed: int, C: int, F: int) -> BlockWeights:
    """Seeded block parameters, all from the BLOCK stream in a fixed order:
    norm gains 1 + 0.1 z, biases 0.1 z, projections z / sqrt(fan-in)
    (rounded to bf16), depthwise taps z / 3."""
    sizes = [C, C, C * C, 9 * C, C, C, C, F * C, F, C * F, C]
    z = normals(seed, STREAM_BLOCK, sum(sizes))
    parts, o = [], 0
    for n in sizes:
        parts.append(z[o:o + n])
        o += n
    f32 = np.float32
    return BlockWeights(
        ln1_w=(1.0 + 0.1 * parts[0]).astype(f32),
        ln1_b=(0.1 * parts[1]).astype(f32),
        wq=round_bf16((parts[2] / math.sqrt(C)).astype(f32).reshape(C, C))[0],
        dw_w=(parts[3] / 3.0).astype(f32).reshape(C, 3, 3),
        dw_b=(0.1 * parts[4]).astype(f32),
        ln2_w=(1.0 + 0.1 * parts[5]).astype(f32),
        ln2_b=(0.1 * parts[6]).astype(f32),
        w1=round_bf16((parts[7] / math.sqrt(C)).astype(f32).reshape(F, C))[0],
        b1=(0.1 * parts[8]).astype(f32),
        w2=round_bf16((parts[9] / math.sqrt(F)).astype(f32).reshape(C, F))[0],
        b2=(0.1 * parts[10]).astype(f32))


@dataclasses.dataclass
class Workload:
    """One synthetic grid. x is kept as fp32 values that are exactly
    representable in ``dtype`` (bf16 values are already rounded)."""
    name: str
    B: int
    H: int
    W: int
    C: int
    heads: int
    d: int
    dtype: str              # "f32" or "bf16"
    x: np.ndarray           # [B,H,W,C] fp32 (bf16-exact when dtype == "bf16")
    states: np.ndarray      # [4][heads][3d^2+2d] fp32
    scales: np.ndarray      # [4][C] fp32
    q: Optional[np.ndarray] = None
    alpha_max: float = 0.9
    eps: float = 1e-6
    chunk_row: int = 0
    chunk_col: int = 0
    route_mask: int = 15
    seed: int = 0

    @property
    def N(self) -> int:
        return self.H * self.W

    def x_words(self) -> np.ndarray:
        """x in its storage dtype: fp32 array, or uint16 bf16 words."""
        if self.dtype == "bf16":
            return round_bf16(self.x)[1]
        return self.x


def _x_normal(seed, B, H, W, C):
    return normals(seed, STREAM_X, B * H * W * C).reshape(B, H, W, C)


def _x_ar1_rows(seed, B, H, W, C, rho):
    z = _x_normal(seed, B, H, W, C)
    x = np.empty_like(z)
    x[:, :, 0, :] = z[:, :, 0, :]
    s = math.sqrt(1.0 - rho * rho)
    for j in range(1, W):
        x[:, :, j, :] = rho * x[:, :, j - 1, :] + s * z[:, :, j, :]
    return x


def outlier_tokens(seed: int, n_tokens: int, frac: float) -> np.ndarray:
    """round(frac * n_tokens) distinct token indices chosen by a partial
    Fisher-Yates shuffle driven by the OUTLIERS stream."""
    m = int(round(frac * n_tokens))
    u = uniforms(seed, STREAM_OUTLIERS, m)
    perm = np.arange(n_tokens, dtype=np.int64)
    for i in range(m):
        j = i + min(int(u[i] * (n_tokens - i)), n_tokens - i - 1)
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:m])


def make(name: str, B, H, W, C, heads, d, dtype, seed, *, x_kind="normal",
         rho=0.9, outlier_frac=0.0, outlier_scale=50.0, state_std=0.02,
         alpha_max=0.9, separate_q=False, chunk_row=0, chunk_col=0,
         route_mask=15) -> Workload:
    if x_kind == "normal":
        x = _x_normal(seed, B, H, W, C)
    elif x_kind == "ar1":
        x = _x_ar1_rows(seed, B, H, W, C, rho)
    elif x_kind == "zero":
        x = np.zeros((B, H, W, C))
    else:
        raise ValueError(x_kind)
    x = x.astype(np.float32)
    if outlier_frac > 0:
        idx = outlier_tokens(seed, B * H * W, outlier_frac)
        flat = x.reshape(B * H * W, C)
        flat[idx] *= np.float32(outlier_scale)
    q = None
    if separate_q:
        q = normals(seed, STREAM_Q, B * H * W * C).reshape(B, H, W, C).astype(np.float32)
    if dtype == "bf16":
        x = round_bf16(x)[0]
        if q is not None:
            q = round_bf16(q)[0]
    st = states(seed, heads, d, state_std)
    sc = scales(seed, C)
    return Workload(name, B, H, W, C, heads, d, dtype, x, st, sc, q=q,
                    alpha_max=alpha_max, chunk_row=chunk_row,
                    chunk_col=chunk_col, route_mask=route_mask, seed=seed)


# The five workloads: the tiny fp32 case, the plain backbone's 14x14 map, the
# hierarchical stage-1 map with row-correlated tokens, the hierarchical stage
# sweep, and the dense-prediction map with x50 outlier tokens.
def tiny() -> Workload:
    return make("tiny_8x8", 1, 8, 8, 16, 1, 16, "f32", 0)


def plain14(B: int = 32) -> Workload:
    return make("plain14", B, 14, 14, 192, 3, 64, "bf16", 1)


def hier56(B: int = 64) -> Workload:
    return make("hier56", B, 56, 56, 64, 2, 32, "bf16", 2, x_kind="ar1", rho=0.9)


def hier56_live(B: int = 64) -> Workload:
    """hier56's launch shape and input (AR(1) rows, seed 2) on states of std 1
    with retention fixed at alpha_max = 0.999 (run with the fixed-retention
    flag): the memories stay O(1) over all 56 chunks of every route."""
    return make("hier56_live", B, 56, 56, 64, 2, 32, "bf16", 2, x_kind="ar1", rho=0.9,
                state_std=1.0, alpha_max=0.999)


def hier_sweep(B: int = 64) -> List[Workload]:
    stages = [(56, 64, 2), (28, 128, 4), (14, 256, 8), (7, 512, 16)]
    return [make(f"hier_sweep_{s}x{s}", B, s, s, C, h, 32, "bf16", 3)
            for s, C, h in stages]


def dense200x304(B: int = 2) -> Workload:
    return make("dense200x304", B, 200, 304, 64, 2, 32, "bf16", 4,
                outlier_frac=0.05, outlier_scale=50.0)
