"""Pins for the block oracle (oracle/block.py), CPU only.

Each part is checked against something other than itself: the layer norm's
defining moments and PyTorch's float64 layer_norm; the depthwise convolution
against PyTorch's grouped conv2d and against delta and shift kernels; GELU
against PyTorch's exact GELU and its reflection identity; and the block's
wiring by special cases that remove one term at a time.
"""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import block as OB
from self_referential_memory_amd import synth


def _rng(seed):
    return np.random.default_rng(seed)


def test_layer_norm_moments_and_library():
    x = _rng(0).standard_normal((3, 5, 7, 24)) * 3.0 + 1.5
    eps = 1e-5
    y = OB.layer_norm(x, np.ones(24), np.zeros(24), eps)
    var = x.var(axis=-1)
    assert np.abs(y.mean(axis=-1)).max() < 1e-14
    assert np.allclose(y.var(axis=-1), var / (var + eps), rtol=1e-13, atol=0)
    w = _rng(1).standard_normal(24)
    b = _rng(2).standard_normal(24)
    ref = F.layer_norm(torch.tensor(x), (24,), torch.tensor(w), torch.tensor(b), eps).numpy()
    assert np.abs(OB.layer_norm(x, w, b, eps) - ref).max() < 1e-13


def test_dwconv_matches_grouped_conv2d():
    B, H, W, C = 2, 5, 6, 8
    u = _rng(3).standard_normal((B, H, W, C))
    w = _rng(4).standard_normal((C, 3, 3))
    b = _rng(5).standard_normal(C)
    ref = F.conv2d(torch.tensor(u).permute(0, 3, 1, 2), torch.tensor(w)[:, None], torch.tensor(b),
                   padding=1, groups=C).permute(0, 2, 3, 1).numpy()
    assert np.abs(OB.dwconv3x3(u, w, b) - ref).max() < 1e-13


def test_dwconv_delta_and_shift_kernels():
    u = _rng(6).standard_normal((1, 4, 5, 3))
    w = np.zeros((3, 3, 3))
    w[:, 1, 1] = 1.0
    assert np.array_equal(OB.dwconv3x3(u, w, np.zeros(3)), u)
    w = np.zeros((3, 3, 3))
    w[:, 0, 1] = 1.0          # tap above: out[i, j] = u[i - 1, j]
    out = OB.dwconv3x3(u, w, np.zeros(3))
    assert np.array_equal(out[:, 1:], u[:, :-1])
    assert np.array_equal(out[:, 0], np.zeros_like(out[:, 0]))
    w = np.zeros((3, 3, 3))
    w[:, 1, 2] = 1.0          # tap to the right: out[i, j] = u[i, j + 1]
    out = OB.dwconv3x3(u, w, np.zeros(3))
    assert np.array_equal(out[:, :, :-1], u[:, :, 1:])
    assert np.array_equal(out[:, :, -1], np.zeros_like(out[:, :, -1]))


def test_gelu_library_and_identities():
    z = np.linspace(-8, 8, 1001)
    ref = F.gelu(torch.tensor(z), approximate="none").numpy()
    assert np.abs(OB.gelu(z) - ref).max() < 1e-15
    assert OB.gelu(0.0) == 0.0
    assert np.allclose(OB.gelu(-z), OB.gelu(z) - z, rtol=0, atol=1e-14)
    assert abs(OB.gelu(1.0) - 0.8413447460685429) < 1e-15   # Phi(1) = 0.841344746068543


def _case(seed=8, H=4, W=5, C=16, heads=2, d=8, F_=32):
    wl = synth.make("blk", 2, H, W, C, heads, d, "f32", seed, state_std=0.5)
    bw = synth.block_weights(seed, C, F_)
    return wl, bw


def test_block_without_ffn_hidden_is_h_plus_output_bias():
    wl, bw = _case()
    bw0 = dataclasses.replace(bw, w1=np.zeros_like(bw.w1), b1=np.zeros_like(bw.b1))
    p = OB.block_forward(wl.x, wl.states, wl.scales, bw0, wl.heads, wl.d, parts=True)
    assert np.array_equal(p["out"], p["h"] + bw.b2.astype(np.float64))


def test_block_without_mixing_branches_keeps_x():
    wl, bw = _case()
    bw0 = dataclasses.replace(bw, dw_w=np.zeros_like(bw.dw_w), dw_b=np.zeros_like(bw.dw_b))
    p = OB.block_forward(wl.x, wl.states, np.zeros_like(wl.scales), bw0, wl.heads, wl.d,
                         parts=True)
    assert np.array_equal(p["h"], wl.x.astype(np.float64))


def test_block_identity_query_projection_is_operator_on_u():
    """With Wq = I the queries are u itself, which is the operator's own
    default (q = x of the scan)."""
    wl, bw = _case()
    bwi = dataclasses.replace(bw, wq=np.eye(wl.C, dtype=np.float32))
    p = OB.block_forward(wl.x, wl.states, wl.scales, bwi, wl.heads, wl.d, parts=True)
    y = oracle.scan(p["u"], wl.states, wl.heads, wl.d, 15)
    assert np.abs(p["y"] - y).max() <= 1e-14 * np.abs(y).max()


def test_block_matches_torch_composition():
    """The whole block against the same wiring written with PyTorch's float64
    layer_norm, grouped conv2d, linear and exact GELU around the C oracle."""
    wl, bw = _case(seed=9)
    out = OB.block_forward(wl.x, wl.states, wl.scales, bw, wl.heads, wl.d)
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    x = t(wl.x)
    C = wl.C
    u = F.layer_norm(x, (C,), t(bw.ln1_w), t(bw.ln1_b), bw.ln_eps)
    q = F.linear(u, t(bw.wq))
    y = oracle.scan(u.numpy(), wl.states, wl.heads, wl.d, 15, q.numpy())
    s = t(oracle.fuse(y, wl.B, wl.H, wl.W, C, 15, wl.scales))
    c = F.conv2d(u.permute(0, 3, 1, 2), t(bw.dw_w)[:, None], t(bw.dw_b), padding=1,
                 groups=C).permute(0, 2, 3, 1)
    h = x + c + s
    v = F.layer_norm(h, (C,), t(bw.ln2_w), t(bw.ln2_b), bw.ln_eps)
    ref = h + F.linear(F.gelu(F.linear(v, t(bw.w1), t(bw.b1))), t(bw.w2), t(bw.b2))
    assert np.abs(out - ref.numpy()).max() <= 1e-12 * np.abs(ref.numpy()).max()


@pytest.mark.parametrize("seed", [1, 2])
def test_block_weights_are_bf16_exact_where_stated(seed):
    bw = synth.block_weights(seed, 32, 128)
    for a in (bw.wq, bw.w1, bw.w2):
        assert np.array_equal(synth.round_bf16(a)[0], a)
