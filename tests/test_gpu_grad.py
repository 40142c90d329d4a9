"""GPU parity of the backward pass: srnl_scan_bwd and srnl_fuse_bwd (through
the C ABI) against the reference gradients of oracle/srnl_grad.py on the same
seeded inputs.

Bar: max |gpu - ref| / max |ref| <= 1e-3 for every gradient (dx, dq, the
initial states, the scales). The gradient runs the fp32 recurrence backwards
through every token of the chain, so it is a longer fp32 computation than
the forward (whose bar is 1e-4).
"""
import numpy as np
import pytest
import torch

from oracle import srnl_grad as G
from self_referential_memory_amd import srnl, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-3

_CAP = {0: G.CAP_SOFT, srnl.FLAG_HARD_CAP: G.CAP_HARD, srnl.FLAG_NO_CAP: G.CAP_OFF}


def _kw(wl, flags):
    return dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
                chunk_col=wl.chunk_col, cap_mode=_CAP[flags & 0x3],
                clamp=not (flags & srnl.FLAG_NO_CLAMP),
                fixed_alpha=bool(flags & srnl.FLAG_FIXED_ALPHA),
                readout_before=bool(flags & srnl.FLAG_READ_BEFORE),
                freeze_kv=bool(flags & srnl.FLAG_FREEZE_KV))


def rel(g, o):
    m = np.abs(o).max()
    return float(np.abs(g - o).max() / m) if m > 0 else float(np.abs(g).max())


def run_case(wl, mask=15, flags=0, seed=0):
    """Full chain on the GPU: scan_fwd, fuse; then fuse_bwd and scan_bwd for
    dL/dfused = dout, plus a direct dL/dy term; against autograd."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    R = bin(mask).count("1")
    print(f"[gpu] grad {wl.name} B={wl.B} {wl.H}x{wl.W} C={wl.C} {wl.heads}x{wl.d} "
          f"mask={mask} flags={flags} chunks=({wl.chunk_row},{wl.chunk_col}) "
          f"q={wl.q is not None}", flush=True)
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((wl.B, wl.H, wl.W, wl.C)).astype(np.float32)
    dyd = rng.standard_normal((R, wl.B, wl.N, wl.C)).astype(np.float32)
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    q = None if wl.q is None else torch.from_numpy(wl.q).to(DEV).to(dt)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col, flags=flags)
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, mask, q, **kw)
    dyr, dsc = srnl.fuse_bwd(torch.from_numpy(dout).to(DEV), y, wl.B, wl.H, wl.W, wl.C, mask, sc)
    dy = dyr + torch.from_numpy(dyd).to(DEV)
    dx, dq, dst = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, mask, q, **kw)
    torch.cuda.synchronize()
    gx, gq, gst, gsc = G.grads(wl.x, wl.states, wl.scales, wl.heads, wl.d, mask, wl.q,
                               dy=dyd, dfused=dout, **_kw(wl, flags))
    got = dict(dx=dx.cpu().numpy(), dst=dst.cpu().numpy(), dsc=dsc.cpu().numpy())
    ref = dict(dx=gx, dst=gst, dsc=gsc)
    if wl.q is not None:
        got["dq"], ref["dq"] = dq.cpu().numpy(), gq
    for k in got:
        assert np.isfinite(got[k]).all(), k
        e = rel(got[k], ref[k])
        assert e <= TOL, (k, e)
    return got, ref


def _wl(name, B, H, W, heads, d, dtype="f32", seed=1, **kw):
    return synth.make(name, B, H, W, heads * d, heads, d, dtype, seed, **kw)


@pytest.mark.parametrize("d,heads", [(4, 2), (8, 2), (16, 2), (32, 2), (64, 1)])
def test_grad_head_dims(d, heads):
    run_case(_wl(f"g{d}", 2, 5, 6, heads, d, seed=d, state_std=0.3))


def test_grad_tiny_workload():
    run_case(synth.tiny())


@pytest.mark.parametrize("flags", [srnl.FLAG_HARD_CAP, srnl.FLAG_NO_CAP, srnl.FLAG_NO_CLAMP,
                                   srnl.FLAG_FIXED_ALPHA, srnl.FLAG_READ_BEFORE,
                                   srnl.FLAG_FREEZE_KV])
def test_grad_variants(flags):
    std = 0.3 if flags == srnl.FLAG_NO_CAP else 1.0
    run_case(_wl("gv", 2, 4, 5, 2, 16, seed=flags, state_std=std), flags=flags)


def test_grad_stressed_inputs_cap_and_clamp_active():
    run_case(_wl("gadv", 1, 6, 5, 2, 16, seed=9, state_std=3.0, outlier_frac=0.1))


@pytest.mark.parametrize("cr,cc", [(3, 2), (1, 1), (7, 0), (100, 100)])
def test_grad_chunk_overrides(cr, cc):
    run_case(_wl("gch", 1, 5, 7, 2, 8, seed=cr * 10 + cc, state_std=0.5,
                 chunk_row=cr, chunk_col=cc))


@pytest.mark.parametrize("mask", [1, 2, 4, 8, 5, 10])
def test_grad_route_masks(mask):
    run_case(_wl("gm", 2, 4, 6, 1, 16, seed=mask), mask=mask)


def test_grad_separate_queries_and_bf16():
    run_case(_wl("gq", 2, 6, 6, 2, 32, dtype="bf16", seed=4, separate_q=True))


def test_grad_d32_long_rows():
    """A 6x40 map at d = 32: row chunks of 40 tokens span two sub-blocks of
    the backward (32 + 8)."""
    run_case(_wl("glong", 1, 6, 40, 2, 32, seed=6, x_kind="ar1"))


# d = 32 without FLAG_READ_BEFORE takes the windowed backward (a forward
# record, then 16-token windows on MFMA); the same cases as above there.
@pytest.mark.parametrize("flags", [0, srnl.FLAG_HARD_CAP, srnl.FLAG_NO_CAP, srnl.FLAG_NO_CLAMP,
                                   srnl.FLAG_FIXED_ALPHA, srnl.FLAG_READ_BEFORE,
                                   srnl.FLAG_FREEZE_KV,
                                   srnl.FLAG_FREEZE_KV | srnl.FLAG_READ_BEFORE])
def test_grad_variants_d32(flags):
    std = 0.3 if flags == srnl.FLAG_NO_CAP else 1.0
    run_case(_wl("gv32", 2, 5, 7, 2, 32, seed=40 + flags, state_std=std), flags=flags)


def test_grad_stressed_inputs_d32():
    run_case(_wl("gadv32", 1, 6, 9, 2, 32, seed=19, state_std=2.0, outlier_frac=0.1))


@pytest.mark.parametrize("cr,cc", [(3, 2), (1, 1), (17, 0), (40, 5), (100, 100)])
def test_grad_chunk_overrides_d32(cr, cc):
    run_case(_wl("gch32", 1, 6, 23, 1, 32, seed=cr * 7 + cc, state_std=0.5,
                 chunk_row=cr, chunk_col=cc))


@pytest.mark.parametrize("mask", [1, 2, 4, 8, 6, 9])
def test_grad_route_masks_d32(mask):
    run_case(_wl("gm32", 2, 4, 6, 1, 32, seed=50 + mask), mask=mask)


def test_grad_separate_queries_f32_d32():
    run_case(_wl("gq32", 2, 5, 6, 2, 32, dtype="f32", seed=8, separate_q=True))


# d = 64 without FLAG_READ_BEFORE, when no route's chunk is longer than 16
# tokens, takes the single-window windowed backward (one 16-token window per
# chunk, Q_0 = I); longer chunks and reading before the write take the
# sequential adjoint.
def test_grad_d64_plain14_map():
    """The plain backbone's map: 14x14, C = 192, 3 heads x d = 64, bf16, four
    routes, 14-token chunks."""
    run_case(_wl("gp14", 1, 14, 14, 3, 64, dtype="bf16", seed=61, x_kind="ar1"))


@pytest.mark.parametrize("flags", [srnl.FLAG_HARD_CAP, srnl.FLAG_NO_CAP, srnl.FLAG_NO_CLAMP,
                                   srnl.FLAG_FIXED_ALPHA, srnl.FLAG_FREEZE_KV,
                                   srnl.FLAG_READ_BEFORE])
def test_grad_variants_d64(flags):
    std = 0.3 if flags == srnl.FLAG_NO_CAP else 1.0
    run_case(_wl("gv64", 2, 5, 7, 1, 64, seed=70 + flags, state_std=std), flags=flags)


def test_grad_stressed_inputs_d64():
    run_case(_wl("gadv64", 1, 7, 9, 2, 64, seed=79, state_std=2.0, outlier_frac=0.1))


@pytest.mark.parametrize("cr,cc", [(5, 3), (1, 1), (16, 16), (17, 4)])
def test_grad_chunk_overrides_d64(cr, cc):
    """Ragged chunks inside one window, one-token chunks, full windows, and a
    17-token row chunk (the sequential adjoint)."""
    run_case(_wl("gch64", 1, 6, 19, 1, 64, seed=cr * 7 + cc, state_std=0.5,
                 chunk_row=cr, chunk_col=cc))


@pytest.mark.parametrize("mask", [1, 2, 4, 8, 6, 9])
def test_grad_route_masks_d64(mask):
    run_case(_wl("gm64", 2, 4, 6, 1, 64, seed=80 + mask), mask=mask)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_separate_queries_d64(dtype):
    run_case(_wl("gq64", 2, 5, 6, 2, 64, dtype=dtype, seed=90, separate_q=True))


def test_grad_is_deterministic():
    wl = _wl("gdet", 2, 5, 5, 2, 16, seed=3)
    a, _ = run_case(wl)
    b, _ = run_case(wl)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_scan_bwd_workspace_errors():
    x = torch.zeros((1, 2, 2, 8), device=DEV)
    st = torch.zeros((4, 2, 3 * 16 + 8), device=DEV)
    p = srnl.make_params(st, x)
    n = srnl.lib().srnl_scan_bwd_workspace_bytes(1, 2, 2, 8, 2, 4, 15, p)
    assert n > 0
    dy = torch.zeros((4, 1, 4, 8), device=DEV)
    dx = torch.empty_like(x)
    dst = torch.empty_like(st)
    ws = torch.empty(n - 4, dtype=torch.uint8, device=DEV)
    import ctypes
    rc = srnl.lib().srnl_scan_bwd(x.data_ptr(), 1, 2, 2, 8, 2, 4, 15, ctypes.byref(p),
                                  dy.data_ptr(), ws.data_ptr(), n - 4, dx.data_ptr(), None,
                                  dst.data_ptr())
    assert rc == srnl.SRNL_ERR_WORKSPACE


def test_grad_hier56_full_map():
    """The benchmark's map at full size (56x56, C=64, 2 heads x d=32, four
    routes, AR(1) rows, bf16 input) on two batch items."""
    run_case(synth.make("hier56_b2", 2, 56, 56, 64, 2, 32, "bf16", 2, x_kind="ar1"))


@pytest.mark.parametrize("dtype,separate_q", [("f32", False), ("bf16", True)])
def test_autograd_operator(dtype, separate_q):
    """srnl.operator under torch.autograd: the forward equals srnl.forward
    bitwise, and the gradients of x, q, the states and the scales equal the
    oracle's for the same output gradient (bf16 gradients of bf16 inputs to
    one bf16 rounding plus the fp32 bar)."""
    wl = _wl("gauto", 2, 5, 6, 2, 32, dtype=dtype, seed=9, separate_q=separate_q)
    print(f"[gpu] autograd {dtype} q={separate_q}", flush=True)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col)
    x = torch.from_numpy(wl.x).to(DEV).to(dt).requires_grad_()
    q = None if wl.q is None else torch.from_numpy(wl.q).to(DEV).to(dt).requires_grad_()
    st = torch.from_numpy(wl.states).to(DEV).requires_grad_()
    sc = torch.from_numpy(wl.scales).to(DEV).requires_grad_()
    out = srnl.operator(x, st, sc, wl.heads, wl.d, 15, q, **kw)
    with torch.no_grad():
        ref_out = srnl.forward(x.detach(), st.detach(), sc.detach(), wl.heads, wl.d, 15,
                               None if q is None else q.detach(), **kw)
    assert out.dtype == dt and torch.equal(out, ref_out)
    g = torch.from_numpy(np.random.default_rng(9).standard_normal(out.shape)
                         .astype(np.float32)).to(DEV).to(dt)
    out.backward(g)
    torch.cuda.synchronize()
    R = 4
    gx, gq, gst, gsc = G.grads(wl.x, wl.states, wl.scales, wl.heads, wl.d, 15, wl.q,
                               dy=np.zeros((R, wl.B, wl.N, wl.C), np.float32),
                               dfused=g.float().cpu().numpy(), **_kw(wl, 0))

    def close(got, ref, name):
        got = got.float().cpu().numpy()
        if dt == torch.bfloat16 and name in ("dx", "dq"):
            bound = 2.0 ** -8 * np.abs(ref) + TOL * np.abs(ref).max()
            assert (np.abs(got - ref) <= bound).all(), name
        else:
            assert rel(got, ref) <= TOL, name

    assert x.grad.dtype == dt
    close(x.grad, gx, "dx")
    close(st.grad, gst, "dst")
    close(sc.grad, gsc, "dsc")
    if q is not None:
        close(q.grad, gq, "dq")


def test_grad_hier56_bench_launch_sampled_items():
    """The backward in the benchmark's launch configuration (56x56, B = 64,
    C = 64, 2 heads x d = 32, bf16, four routes). dx of items 0 and 63 is
    checked against the oracle on those items. The state and scale
    gradients are sums over the batch; by linearity in the output gradient,
    the full run's minus that of a second run whose output gradient is zero
    on items 0 and 63 is the two items' share, checked against the oracle."""
    wl = synth.hier56()
    print(f"[gpu] grad hier56 B={wl.B} sampled items", flush=True)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col)
    x = torch.from_numpy(wl.x).to(DEV).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    sel = [0, wl.B - 1]
    dout = np.random.default_rng(11).standard_normal((wl.B, wl.H, wl.W, wl.C)).astype(np.float32)
    rest = dout.copy()
    rest[sel] = 0.0
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, 15, **kw)
    out = []
    for g in (dout, rest):
        dyr, dsc = srnl.fuse_bwd(torch.from_numpy(g).to(DEV), y, wl.B, wl.H, wl.W, wl.C, 15, sc)
        dx, _, dst = srnl.scan_bwd(x, st, wl.heads, wl.d, dyr, 15, **kw)
        out.append((dx.cpu().numpy(), dst.cpu().numpy().astype(np.float64),
                    dsc.cpu().numpy().astype(np.float64)))
    torch.cuda.synchronize()
    gx, _, gst, gsc = G.grads(wl.x[sel], wl.states, wl.scales, wl.heads, wl.d, 15, None,
                              dy=np.zeros((4, 2, wl.N, wl.C), np.float32), dfused=dout[sel],
                              **_kw(wl, 0))
    assert np.isfinite(out[0][0]).all()
    assert rel(out[0][0][sel], gx) <= TOL, "dx"
    assert rel(out[0][1] - out[1][1], gst) <= TOL, "dstates"
    assert rel(out[0][2] - out[1][2], gsc) <= TOL, "dscales"
    assert not out[1][0][sel].any()     # zero output gradient, zero dx


def test_backward_on_a_side_stream_matches():
    """The backward entry points and the block launched on a stream other
    than the current one (the binding's temporaries are recorded on it)
    give bitwise the results of the current-stream calls."""
    print("[gpu] side-stream backward and block", flush=True)
    wl = _wl("gside", 2, 6, 7, 2, 32, dtype="bf16", seed=12)
    x = torch.from_numpy(wl.x).to(DEV).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps)
    dout = torch.from_numpy(np.random.default_rng(12).standard_normal(
        (wl.B, wl.H, wl.W, wl.C)).astype(np.float32)).to(DEV)
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, 15, **kw)
    ref_dy, ref_dsc = srnl.fuse_bwd(dout, y, wl.B, wl.H, wl.W, wl.C, 15, sc)
    ref = srnl.scan_bwd(x, st, wl.heads, wl.d, ref_dy, 15, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    dy, dsc = srnl.fuse_bwd(dout, y, wl.B, wl.H, wl.W, wl.C, 15, sc, stream=side)
    side.synchronize()
    got = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15, stream=side, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dy, ref_dy) and torch.equal(dsc, ref_dsc)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[2], ref[2])


@pytest.mark.parametrize("case", ["hier", "long_q_f32", "ragged_q_f32", "short_chunks", "t32",
                                  "variants", "fixed_alpha", "plain14_d64", "ragged_q_d64"])
def test_forward_record_matches(case):
    """SRNL_FLAG_RECORD: the forward that keeps its record gives the plain
    forward's outputs bitwise, and the backward that reads that record gives
    bitwise the gradients of the backward that records by itself."""
    flags = 0
    if case == "hier":
        wl = _wl("rec_h", 2, 56, 56, 2, 32, dtype="bf16", seed=21)
    elif case == "long_q_f32":
        wl = _wl("rec_l", 2, 40, 40, 2, 32, dtype="f32", seed=29, separate_q=True)
    elif case == "ragged_q_f32":
        wl = _wl("rec_q", 2, 9, 13, 2, 32, dtype="f32", seed=22, separate_q=True,
                 chunk_row=5, chunk_col=4)
    elif case == "short_chunks":
        wl = _wl("rec_s", 3, 7, 7, 2, 32, dtype="bf16", seed=23)
    elif case == "t32":
        wl = _wl("rec_t", 2, 28, 20, 2, 32, dtype="bf16", seed=24)
    elif case == "variants":
        wl = _wl("rec_v", 2, 12, 17, 2, 32, dtype="f32", seed=25, state_std=2.0,
                 outlier_frac=0.05)
        flags = srnl.FLAG_HARD_CAP | srnl.FLAG_NO_CLAMP | srnl.FLAG_FREEZE_KV
    elif case == "plain14_d64":
        wl = _wl("rec_p", 2, 14, 14, 3, 64, dtype="bf16", seed=31)
    elif case == "ragged_q_d64":
        wl = _wl("rec_r", 2, 9, 13, 1, 64, dtype="f32", seed=32, separate_q=True,
                 chunk_row=5, chunk_col=4)
        flags = srnl.FLAG_FREEZE_KV
    else:
        wl = _wl("rec_a", 2, 10, 11, 2, 32, dtype="bf16", seed=26)
        flags = srnl.FLAG_FIXED_ALPHA
    print(f"[gpu] record {case} {wl.B}x{wl.H}x{wl.W} flags={flags}", flush=True)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    q = None if wl.q is None else torch.from_numpy(wl.q).to(DEV).to(dt)
    st = torch.from_numpy(wl.states).to(DEV)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col, flags=flags)
    y0 = srnl.scan_fwd(x, st, wl.heads, wl.d, 15, q, **kw)
    y1, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15, q, **kw)
    assert rec is not None
    dy = torch.from_numpy(np.random.default_rng(7).standard_normal(tuple(y0.shape))
                          .astype(np.float32)).to(DEV)
    g0 = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15, q, **kw)
    g1 = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15, q, record=rec, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for a, b in zip(g0, g1):
        assert (a is None and b is None) or torch.equal(a, b)


def test_forward_record_where_it_does_not_apply_and_errors():
    """d = 16, d = 64 with chunks longer than 16 tokens and the readout-
    before-write variant have no record: the forward runs plainly and the
    binding returns None. A record smaller than the sizes need is a workspace
    error in both directions."""
    print("[gpu] record n/a and errors", flush=True)
    wl = _wl("rec_n", 2, 5, 6, 2, 16, dtype="f32", seed=27)
    x = torch.from_numpy(wl.x).to(DEV)
    st = torch.from_numpy(wl.states).to(DEV)
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15)
    assert rec is None and torch.equal(y, srnl.scan_fwd(x, st, wl.heads, wl.d, 15))
    # d = 64 with a route's chunks longer than one window: no record either
    wl = _wl("rec_n64", 1, 4, 17, 1, 64, dtype="f32", seed=30)
    x = torch.from_numpy(wl.x).to(DEV)
    st = torch.from_numpy(wl.states).to(DEV)
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15)
    assert rec is None and torch.equal(y, srnl.scan_fwd(x, st, wl.heads, wl.d, 15))
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15, chunk_row=16)
    assert rec is not None
    wl = _wl("rec_e", 2, 5, 6, 2, 32, dtype="f32", seed=28)
    x = torch.from_numpy(wl.x).to(DEV)
    st = torch.from_numpy(wl.states).to(DEV)
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15, flags=srnl.FLAG_READ_BEFORE)
    assert rec is None
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15)
    p = srnl.make_params(st, x, flags=srnl.FLAG_RECORD)
    p.workspace, p.workspace_bytes = rec.data_ptr(), rec.numel() - 256
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd(x, st, wl.heads, wl.d, 15, params=p)
    assert e.value.status == srnl.SRNL_ERR_WORKSPACE
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_bwd(x, st, wl.heads, wl.d, torch.zeros_like(y), 15, record=rec[:-256])
    assert e.value.status == srnl.SRNL_ERR_WORKSPACE


def test_forward_record_with_finite_check():
    """SRNL_FLAG_RECORD with SRNL_FLAG_CHECK_FINITE: the counters sit after
    the record in the one workspace; the record still serves the backward,
    and a NaN input is still reported."""
    print("[gpu] record + finite check", flush=True)
    wl = _wl("rec_f", 2, 9, 10, 2, 32, dtype="bf16", seed=30)
    x = torch.from_numpy(wl.x).to(DEV).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(DEV)
    y0 = srnl.scan_fwd(x, st, wl.heads, wl.d, 15)
    y1, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15, flags=srnl.FLAG_CHECK_FINITE)
    dy = torch.from_numpy(np.random.default_rng(8).standard_normal(tuple(y0.shape))
                          .astype(np.float32)).to(DEV)
    g0 = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15)
    g1 = srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15, record=rec)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(g0[0], g1[0]) and torch.equal(g0[2], g1[2])
    xb = x.clone()
    xb.view(-1)[3] = float("nan")
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd_record(xb, st, wl.heads, wl.d, 15, flags=srnl.FLAG_CHECK_FINITE)
    assert e.value.status == srnl.SRNL_ERR_NONFINITE
    assert "1 non-finite input values" in str(e.value)


@pytest.mark.parametrize("chunk,record,dtype,separate_q", [
    (0, True, "bf16", False), (0, False, "f32", False), (100, True, "f32", True)])
def test_scan_1d_backward_matches_oracle(chunk, record, dtype, separate_q):
    """srnl_scan_1d_bwd after srnl_scan_1d (with the forward keeping its
    record, or the backward recording it itself), 64-token default chunks or
    a 100-token override, 300 tokens (a short final chunk), against the
    gradient oracle on the 1 x N grid's row route; the state gradient comes
    back in the 1-D layout [heads][3d^2+2d]."""
    B, N, C, heads, d = 2, 300, 64, 2, 32
    print(f"[gpu] 1-D backward chunk={chunk} record={record} {dtype} q={separate_q}", flush=True)
    wl = _wl("g1d", B, 1, N, heads, d, dtype=dtype, seed=31, state_std=0.5,
             separate_q=separate_q)
    st1 = np.ascontiguousarray(wl.states[0])
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(wl.x.reshape(B, N, C)).to(DEV).to(dt)
    q = None if wl.q is None else torch.from_numpy(wl.q.reshape(B, N, C)).to(DEV).to(dt)
    st = torch.from_numpy(st1).to(DEV)
    dyd = np.random.default_rng(31).standard_normal((B, N, C)).astype(np.float32)
    dy = torch.from_numpy(dyd).to(DEV)
    if record:
        y, rec = srnl.scan_1d_record(x, st, heads, d, q, chunk=chunk)
        assert rec is not None
    else:
        y, rec = srnl.scan_1d(x, st, heads, d, q, chunk=chunk), None
    dx, dq, dst = srnl.scan_1d_bwd(x, st, heads, d, dy, q, chunk=chunk, record=rec)
    torch.cuda.synchronize()
    assert torch.equal(y, srnl.scan_1d(x, st, heads, d, q, chunk=chunk))
    st4 = np.zeros((4,) + st1.shape, np.float32)
    st4[0] = st1
    gx, gq, gst, _ = G.grads(wl.x, st4, np.ones((4, C), np.float32), heads, d, 1, wl.q,
                             dy=dyd.reshape(1, B, N, C), dfused=None,
                             chunk_row=chunk if chunk > 0 else 64, chunk_col=0)
    assert tuple(dst.shape) == (heads, 3 * d * d + 2 * d)
    assert rel(dx.cpu().numpy(), gx.reshape(B, N, C)) <= TOL, "dx"
    assert rel(dst.cpu().numpy(), gst[0]) <= TOL, "dstates"
    assert not gst[1:].any()
    if q is not None:
        assert rel(dq.cpu().numpy(), gq.reshape(B, N, C)) <= TOL, "dq"
    # the same gradients as the 2-D backward on the 1 x N grid with the chunk
    # spelled out
    dx2, dq2, dst2 = srnl.scan_bwd(x.view(B, 1, N, C), torch.from_numpy(st4).to(DEV), heads, d,
                                   dy.view(1, B, N, C), 1,
                                   None if q is None else q.view(B, 1, N, C),
                                   chunk_row=chunk if chunk > 0 else 64)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2.view(B, N, C)) and torch.equal(dst, dst2[0])


def test_autograd_operator_on_a_side_stream_matches():
    """srnl.operator(..., stream=side): the forward output and every
    gradient equal, bitwise, those of the same node on the current stream.
    The side stream waits for the inputs made on the current stream, and the
    current stream for the results (no synchronisation in between here)."""
    print("[gpu] autograd node on a side stream", flush=True)
    wl = _wl("gauto_side", 2, 9, 11, 2, 32, dtype="bf16", seed=33, separate_q=True)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps)

    def run(stream):
        x = torch.from_numpy(wl.x).to(DEV).to(torch.bfloat16).requires_grad_()
        q = torch.from_numpy(wl.q).to(DEV).to(torch.bfloat16).requires_grad_()
        st = torch.from_numpy(wl.states).to(DEV).requires_grad_()
        sc = torch.from_numpy(wl.scales).to(DEV).requires_grad_()
        out = srnl.operator(x, st, sc, wl.heads, wl.d, 15, q, stream=stream, **kw)
        g = (out.float() * 0.5 + 1.0).to(torch.bfloat16)     # made on the current stream
        out.backward(g)
        return [t.clone() for t in (out, x.grad, q.grad, st.grad, sc.grad)]

    ref = run(None)
    side = torch.cuda.Stream()
    got = run(side)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
