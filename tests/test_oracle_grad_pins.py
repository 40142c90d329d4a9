"""Pins for the reference gradients (oracle/srnl_grad.py), CPU only.

The gradient oracle is autograd over a float64 PyTorch restatement of the
operator. It is pinned to things other than itself:
  * its forward values equal the C oracle's (an independent program) on
    every variant, to 1e-12;
  * its directional derivatives equal central finite differences of the C
    oracle's forward, along random directions in x, q, the initial states
    and the fusion scales, on random and stressed inputs and every variant;
  * with x = 0 and separate queries the outputs have a closed form,
    y_t = (alpha_max / 2)^(t+1) M_c q_t, so the query and content-memory
    gradients do too, and every other state row has zero gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import srnl_grad as G
from self_referential_memory_amd import synth

VARIANTS = [
    dict(),
    dict(chunk_row=2, chunk_col=5),
    dict(cap_mode=G.CAP_HARD),
    dict(cap_mode=G.CAP_OFF, clamp=False),
    dict(clamp=False),
    dict(readout_before=True),
    dict(fixed_alpha=True),
    dict(freeze_kv=True, chunk_row=2, chunk_col=5),
]


def _case(seed, B=1, H=3, W=4, heads=2, d=4, std=0.5, xscale=2.0, q=False):
    wl = synth.make("g", B, H, W, heads * d, heads, d, "f32", seed, state_std=std,
                    separate_q=q)
    x = wl.x.astype(np.float64) * xscale
    qq = None if wl.q is None else wl.q.astype(np.float64)
    return x, qq, wl.states.astype(np.float64), wl.scales.astype(np.float64)


def _c_loss(x, q, st, sc, heads, d, dy, df, kw):
    y = oracle.scan(x, st, heads, d, 15, q, **kw)
    B, H, W, C = x.shape
    f = oracle.fuse(y, B, H, W, C, 15, sc)
    return float((y * dy).sum() + (f * df).sum())


@pytest.mark.parametrize("kw", VARIANTS)
def test_torch_forward_equals_c_oracle(kw):
    x, q, st, sc = _case(11, B=2, q=True)
    y, f = G.forward(torch.tensor(x), torch.tensor(st), torch.tensor(sc), 2, 4, 15,
                     torch.tensor(q), **kw)
    yo = oracle.scan(x, st, 2, 4, 15, q, **kw)
    fo = oracle.fuse(yo, 2, 3, 4, 8, 15, sc)
    assert np.abs(y.numpy() - yo).max() <= 1e-12 * np.abs(yo).max()
    assert np.abs(f.numpy() - fo).max() <= 1e-12 * np.abs(fo).max()


@pytest.mark.parametrize("kw", VARIANTS)
@pytest.mark.parametrize("stress", [False, True])
def test_gradients_match_central_differences(kw, stress):
    """<grad, delta> against (L(p + h delta) - L(p - h delta)) / 2h of the C
    oracle, for random directions delta in each input separately."""
    std, xs = (2.0, 3.0) if stress else (0.5, 2.0)
    x, q, st, sc = _case(5 + 3 * stress, std=std, xscale=xs, q=True)
    heads, d = 2, 4
    rng = np.random.default_rng(17)
    dy = rng.standard_normal((4,) + (x.shape[0], x.shape[1] * x.shape[2], x.shape[3]))
    df = rng.standard_normal(x.shape)
    gx, gq, gst, gsc = G.grads(x, st, sc, heads, d, 15, q, dy=dy, dfused=df, **kw)
    h = 1e-6   # truncation error falls as h^2: ~1e-9 relative here; rounding ~1e-9
    for name, base, grad in (("x", x, gx), ("q", q, gq), ("states", st, gst), ("scales", sc, gsc)):
        for _ in range(2):
            delta = rng.standard_normal(base.shape)
            args = {"x": x, "q": q, "st": st, "sc": sc}
            key = {"x": "x", "q": "q", "states": "st", "scales": "sc"}[name]
            lp = dict(args); lp[key] = base + h * delta
            lm = dict(args); lm[key] = base - h * delta
            fd = (_c_loss(lp["x"], lp["q"], lp["st"], lp["sc"], heads, d, dy, df, kw)
                  - _c_loss(lm["x"], lm["q"], lm["st"], lm["sc"], heads, d, dy, df, kw)) / (2 * h)
            an = float((grad * delta).sum())
            assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (name, an, fd)


def test_gradients_zero_input_closed_form():
    """x = 0, separate q: k = v = 0, eta = 1/2, alpha = alpha_max / 2, no
    write, so y_t = a^(t+1) M_c q_t with a = alpha_max / 2 (t counts from the
    start of the scan). Hence dq_t = a^(t+1) M_c^T dy_t, dM_c = sum_t a^(t+1)
    dy_t q_t^T, and every other state row has zero gradient."""
    B, H, W, heads, d = 2, 3, 3, 2, 4
    C = heads * d
    x, q, st, sc = _case(23, B=B, H=H, W=W, heads=heads, d=d, q=True)
    x = np.zeros_like(x)
    rng = np.random.default_rng(3)
    dy = rng.standard_normal((4, B, H * W, C))
    gx, gq, gst, _ = G.grads(x, st, sc, heads, d, 15, q, dy=dy, alpha_max=0.9)
    a = 0.45
    N = H * W
    dq = np.zeros((B, N, C))
    dst = np.zeros_like(st)
    qf = q.reshape(B, N, C)
    for r in range(4):
        order = G.route_order(r, H, W)
        for t in range(N):
            f = a ** (t + 1)
            for hh in range(heads):
                Mc = st[r, hh, :d * d].reshape(d, d)
                sl = slice(hh * d, (hh + 1) * d)
                dq[:, order[t], sl] += f * dy[r, :, t, sl] @ Mc
                dst[r, hh, :d * d] += f * np.einsum("bi,bj->ij", dy[r, :, t, sl],
                                                    qf[:, order[t], sl]).reshape(-1)
    assert np.abs(gq.reshape(B, N, C) - dq).max() <= 1e-12 * np.abs(dq).max()
    assert np.abs(gst - dst).max() <= 1e-12 * np.abs(dst).max()
