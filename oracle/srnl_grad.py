"""TEST INFRASTRUCTURE ONLY: reference gradients of the SRNL forward pass.

A plain float64 PyTorch (CPU) restatement of the operator in its five-memory
form, differentiated by autograd. Only the test suite and the smoke check
may use it. It shares no code with the HIP library, and none with the C
oracle either: it is a second, independent reading of the same passages, so
that the C oracle pins its forward values and central finite differences of
the C oracle pin its gradients.

Sources, cited by page title and section:
  [README]   "VisionHOPE" README: "SRNL and VisionHOPE operator" (training
             with autograd; queries; chunking), "Fast inference".
  [OVERVIEW] "VisionHOPE Model Overview: Architecture, Benchmarks, and
             Practical Limits": "How VisionHOPE's Five Memories Work",
             "Four-Directional Scanning and Spatial Chunking", "Why the
             Stability Controls Matter".
  [SUMMARY]  "VisionHOPE: Visual Backbones as Self-Modifying Learning
             Systems": the paragraphs on the write rule, stabilisation and
             2-D maps.

Per chain (route r, batch item b, head h), with boundary rows B (M_c, M_k,
M_v, m_eta, m_alpha) taken at each chunk start and working memories M:
    k = B_k x, v = B_v x, eta = sigmoid(b_eta . x),
    alpha = alpha_max sigmoid(b_alpha . x)                 [SUMMARY 2-D maps]
    k^ = k / sqrt(|k|^2 + eps), e = k^ - v, g = |e| |k^|   [SUMMARY stabilisation]
    eta' = (1 - alpha) tanh(eta g / (1 - alpha)) / g       (soft cap)
    eta'' = min(eta', 2 alpha / |k^|^2)                    (spectral clamp)
    M <- alpha M - eta'' (M k^ + B e) k^T, row by row      [SUMMARY write rule]
    y_t = M_c q_t after the write                          [README operator]
and the fused map sums scales_r * y_r restored to grid order
[OVERVIEW Four-Directional Scanning and Spatial Chunking]. The same
readings as the C oracle (listed in its header) are taken, including the
ablation variants.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

CAP_SOFT, CAP_HARD, CAP_OFF = 0, 1, 2


def route_order(r: int, H: int, W: int) -> np.ndarray:
    """Grid cell (flattened row-major) that route r visits at each step:
    forward/reverse row-major, forward/reverse column-major
    [OVERVIEW Four-Directional Scanning and Spatial Chunking]."""
    cells = np.arange(H * W).reshape(H, W)
    if r < 2:
        o = cells.reshape(-1)
    else:
        o = cells.T.reshape(-1)
    return o[::-1].copy() if r & 1 else o


def forward(x, states, scales, heads: int, d: int, route_mask: int = 15, q=None, *,
            alpha_max: float = 0.9, eps: float = 1e-6, chunk_row: int = 0,
            chunk_col: int = 0, cap_mode: int = CAP_SOFT, clamp: bool = True,
            fixed_alpha: bool = False, readout_before: bool = False,
            freeze_kv: bool = False):
    """x [B,H,W,C], states [4][heads][3d^2+2d], scales [4][C] (float64
    tensors; q like x or None). Returns (y [R][B][H*W][C] in traversal
    order, fused [B,H,W,C]). ``freeze_kv`` writes only the content memory
    (the frozen key/value and dynamics ablation, [SUMMARY ablation
    paragraph])."""
    B, H, W, C = x.shape
    N = H * W
    routes = [r for r in range(4) if (route_mask >> r) & 1]
    R = len(routes)
    rows = 3 * d + 2
    qsrc = x if q is None else q
    xf = x.reshape(B, N, heads, d)
    qf = qsrc.reshape(B, N, heads, d)
    orders = [torch.as_tensor(route_order(r, H, W)) for r in routes]
    X = torch.stack([xf[:, o] for o in orders])          # [R,B,N,heads,d]
    Q = torch.stack([qf[:, o] for o in orders])
    lens = [(chunk_row if chunk_row > 0 else W) if r < 2 else (chunk_col if chunk_col > 0 else H)
            for r in routes]
    S = states.reshape(4, heads, rows, d)[routes]        # [R,heads,rows,d]
    M = S[:, None].expand(R, B, heads, rows, d)
    Bn = M
    ys = []
    for t in range(N):
        start = torch.tensor([t % L == 0 for L in lens]).view(R, 1, 1, 1, 1)
        Bn = torch.where(start, M, Bn)                   # boundary snapshot
        xt = X[:, :, t]                                  # [R,B,heads,d]
        k = torch.einsum("rbhij,rbhj->rbhi", Bn[..., d:2 * d, :], xt)
        v = torch.einsum("rbhij,rbhj->rbhi", Bn[..., 2 * d:3 * d, :], xt)
        eta = torch.sigmoid((Bn[..., 3 * d, :] * xt).sum(-1))
        if fixed_alpha:
            alpha = torch.full_like(eta, alpha_max)
        else:
            alpha = alpha_max * torch.sigmoid((Bn[..., 3 * d + 1, :] * xt).sum(-1))
        kh = k / torch.sqrt((k * k).sum(-1, keepdim=True) + eps)
        e = kh - v
        nkh2 = (kh * kh).sum(-1)
        pg = (e * e).sum(-1) * nkh2                      # g^2; sqrt kept off 0 for autograd
        g = torch.where(pg > 0, torch.sqrt(torch.where(pg > 0, pg, torch.ones_like(pg))),
                        torch.zeros_like(pg))
        m = 1.0 - alpha
        one = torch.ones_like(g)
        if cap_mode == CAP_SOFT:
            # (1 - alpha) tanh(u) / g with u = eta g / (1 - alpha) is eta tanh(u) / u;
            # written so, with tanh(u)/u's series below u = 1e-4 (its next term
            # is below 1e-25), the derivative has no 1/g^2 cancellation on
            # tiny g; u = 0 (g = 0) gives eta' = eta
            u = eta * g / m
            big = u > 1e-4
            us = torch.where(big, u, one)
            eta1 = eta * torch.where(big, torch.tanh(us) / us,
                                     1.0 - u * u / 3.0 + 2.0 * u ** 4 / 15.0)
        elif cap_mode == CAP_HARD:
            act = (g > 0) & (m < eta * g)
            eta1 = torch.where(act, m / torch.where(act, g, one), eta)
        else:
            eta1 = eta
        if clamp:
            act = (nkh2 > 0) & (2.0 * alpha < eta1 * nkh2)   # 2 alpha / |k^|^2 < eta'
            eta2 = torch.where(act, 2.0 * alpha / torch.where(act, nkh2, one), eta1)
        else:
            eta2 = eta1
        qt = Q[:, :, t]
        if readout_before:
            ys.append(torch.einsum("rbhij,rbhj->rbhi", M[..., :d, :], qt))
        w = torch.einsum("rbhij,rbhj->rbhi", Bn, e)      # B e, every row
        s = torch.einsum("rbhij,rbhj->rbhi", M, kh) + w  # M k^ + B e
        Mw = alpha[..., None, None] * M - eta2[..., None, None] * s[..., None] * kh[..., None, :]
        M = torch.cat([Mw[..., :d, :], M[..., d:, :]], dim=-2) if freeze_kv else Mw
        if not readout_before:
            ys.append(torch.einsum("rbhij,rbhj->rbhi", M[..., :d, :], qt))
    y = torch.stack(ys, dim=2).reshape(R, B, N, C)
    fused = torch.zeros((B, N, C), dtype=y.dtype)
    for s_, (r, o) in enumerate(zip(routes, orders)):
        inv = torch.empty_like(o)
        inv[o] = torch.arange(N)
        fused = fused + scales[r] * y[s_][:, inv]
    return y, fused.reshape(B, H, W, C)


def grads(x, states, scales, heads: int, d: int, route_mask: int = 15, q=None, *,
          dy=None, dfused=None, **kw):
    """Gradients of  sum(dy * y) + sum(dfused * fused)  with respect to x,
    q (None when q = x), states and scales, as float64 numpy arrays.
    Inputs are numpy arrays; dy is [R][B][H*W][C] in traversal order."""
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    st = torch.tensor(np.asarray(states, np.float64), requires_grad=True)
    sc = torch.tensor(np.asarray(scales, np.float64), requires_grad=True)
    qt = None if q is None else torch.tensor(np.asarray(q, np.float64), requires_grad=True)
    y, fused = forward(xt, st, sc, heads, d, route_mask, qt, **kw)
    loss = torch.zeros((), dtype=torch.float64)
    if dy is not None:
        loss = loss + (y * torch.as_tensor(np.asarray(dy, np.float64))).sum()
    if dfused is not None:
        loss = loss + (fused * torch.as_tensor(np.asarray(dfused, np.float64))).sum()
    inputs = [xt, st, sc] + ([qt] if qt is not None else [])
    gs = torch.autograd.grad(loss, inputs, allow_unused=True)
    out = [np.zeros(i.shape) if g is None else g.numpy() for g, i in zip(gs, inputs)]
    dx, dst, dsc = out[:3]
    dq = out[3] if qt is not None else None
    return dx, dq, dst, dsc
