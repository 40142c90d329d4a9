"""TEST INFRASTRUCTURE ONLY: float64 CPU reference of one VisionHOPE residual
block around the four-route SRNL operator.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module. It uses the C oracle (``oracle.scan`` and
``oracle.fuse``) for the operator itself and numpy for the rest; it shares
nothing with the HIP library.

Sources (web pages about VisionHOPE; cited by title and section):
  [SUMMARY]  "VisionHOPE: Visual Backbones as Self-Modifying Learning
             Systems", the paragraph on 2-D maps: the block is a standard
             two-branch residual, a depthwise convolution for local context
             and SRNL for long range, followed by a feed-forward network; and
             the paragraph on what was dropped: the query projection stays
             outside the memory loop.
  [OVERVIEW] "VisionHOPE Model Overview", section "Four-Directional Scanning
             and Spatial Chunking": one shared query projection feeds the
             readout queries of every route, and the backbone's residual
             blocks contain projections, normalisation, a depthwise
             convolution and a feed-forward network.

The pages name the parts but not their exact wiring or sizes. The plainest
consistent reading is taken (each is marked READING and listed in the design
notes):

  u   = LN1(x)                                   normalisation     (READING)
  q   = u Wq^T                                   shared query projection,
                                                 no bias           (READING)
  s   = fuse_r( SRNL_r(u; q) )                   the operator, its input u,
                                                 its queries q
  h   = x + DWConv3x3(u) + s                     two branches, one residual
                                                                   (READING)
  out = h + W2 GELU(W1 LN2(h) + b1) + b2         feed-forward residual,
                                                 exact erf GELU    (READING)

LN is a per-token layer norm over the channels with gain and bias (biased
variance, eps inside the square root). DWConv3x3 is a per-channel 3x3
cross-correlation with zero padding and a bias.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

import oracle


def layer_norm(x, w, b, eps):
    """Per-token layer norm over the last axis: (x - mean) / sqrt(var + eps)
    * w + b, with the biased variance."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(w, np.float64) + np.asarray(b, np.float64)


def dwconv3x3(u, w, b):
    """Depthwise 3x3 cross-correlation with zero padding: out[b,i,j,c] =
    bias[c] + sum_{a,e in {0,1,2}} w[c,a,e] u[b, i+a-1, j+e-1, c]. u is
    [B,H,W,C] (channels last), w is [C][3][3]."""
    u = np.asarray(u, np.float64)
    w = np.asarray(w, np.float64)
    B, H, W, C = u.shape
    pad = np.zeros((B, H + 2, W + 2, C))
    pad[:, 1:H + 1, 1:W + 1] = u
    out = np.broadcast_to(np.asarray(b, np.float64), (B, H, W, C)).copy()
    for a in range(3):
        for e in range(3):
            out += w[:, a, e] * pad[:, a:a + H, e:e + W]
    return out


def gelu(z):
    """Exact GELU: z * Phi(z) = z / 2 * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def block_forward(x, states, scales, bw, heads: int, d: int, route_mask: int = 15,
                  *, threads: int = 1, parts: bool = False, **srnl_kw):
    """One residual block on x [B,H,W,C]. ``bw`` carries the block parameters
    (attributes ln1_w, ln1_b, wq, dw_w, dw_b, ln2_w, ln2_b, w1, b1, w2, b2,
    ln_eps). ``srnl_kw`` goes to the operator (chunks, variants). Returns the
    block output in float64, or with ``parts`` a dict of every intermediate."""
    x = np.asarray(x, np.float64)
    B, H, W, C = x.shape
    f = lambda a: np.asarray(a, np.float64)
    u = layer_norm(x, bw.ln1_w, bw.ln1_b, bw.ln_eps)
    q = u @ f(bw.wq).T
    y = oracle.scan(u, states, heads, d, route_mask, q, threads=threads, **srnl_kw)
    s = oracle.fuse(y, B, H, W, C, route_mask, scales)
    c = dwconv3x3(u, bw.dw_w, bw.dw_b)
    h = x + c + s
    v = layer_norm(h, bw.ln2_w, bw.ln2_b, bw.ln_eps)
    a = v @ f(bw.w1).T + f(bw.b1)
    out = h + gelu(a) @ f(bw.w2).T + f(bw.b2)
    if parts:
        return dict(u=u, q=q, y=y, s=s, c=c, h=h, v=v, a=a, out=out)
    return out
