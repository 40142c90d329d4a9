"""GPU tests of srnl_scan_fuse_bwd, the operator's backward in one call
(through the C ABI): its results are bitwise those of srnl_fuse_bwd followed
by srnl_scan_bwd on the same seeded inputs, both where the windowed d = 32
adjoint forms each route's dy from dout and the scales itself and where the
route gradients go through the workspace; those two calls are checked
against oracle/srnl_grad.py in test_gpu_grad.py, and one case here checks
the one-call path against the oracle directly."""
import numpy as np
import pytest
import torch

from oracle import srnl_grad as G
from self_referential_memory_amd import srnl, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _wl(name, B, H, W, heads, d, dtype="f32", seed=1, **kw):
    return synth.make(name, B, H, W, heads * d, heads, d, dtype, seed, **kw)


def _both(wl, mask=15, flags=0, record=False, seed=0):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    print(f"[gpu] scan_fuse_bwd {wl.name} B={wl.B} {wl.H}x{wl.W} C={wl.C} {wl.heads}x{wl.d} "
          f"mask={mask} flags={flags} chunks=({wl.chunk_row},{wl.chunk_col}) "
          f"q={wl.q is not None} record={record}", flush=True)
    rng = np.random.default_rng(seed)
    dout = torch.from_numpy(rng.standard_normal((wl.B, wl.H, wl.W, wl.C)).astype(np.float32)).to(DEV)
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    q = None if wl.q is None else torch.from_numpy(wl.q).to(DEV).to(dt)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col, flags=flags)
    if record:
        y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, mask, q, **kw)
    else:
        y, rec = srnl.scan_fwd(x, st, wl.heads, wl.d, mask, q, **kw), None
    dyr, dsc0 = srnl.fuse_bwd(dout, y, wl.B, wl.H, wl.W, wl.C, mask, sc)
    dx0, dq0, dst0 = srnl.scan_bwd(x, st, wl.heads, wl.d, dyr, mask, q, record=rec, **kw)
    dx1, dq1, dst1, dsc1 = srnl.scan_fuse_bwd(x, st, wl.heads, wl.d, y, sc, dout, mask, q,
                                              record=rec, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dx0, dx1)
    assert torch.equal(dst0, dst1)
    assert torch.equal(dsc0, dsc1)
    if q is not None:
        assert torch.equal(dq0, dq1)
    return dout, (dx1, dq1, dst1, dsc1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mask", [15, 0b0101, 0b1000])
def test_direct_d32_matches_two_calls(dtype, mask):
    # the windowed d = 32 adjoint reads dout itself: several windows and
    # chunks, a ragged last window
    _both(_wl("sf32", 2, 21, 19, 2, 32, dtype, seed=3, state_std=0.3), mask)


@pytest.mark.parametrize("cr,cc", [(7, 0), (0, 5), (40, 33)])
def test_direct_d32_chunk_overrides(cr, cc):
    _both(_wl("sf32c", 1, 18, 22, 2, 32, "bf16", seed=4, state_std=0.3, chunk_row=cr, chunk_col=cc))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_direct_d32_separate_queries_and_record(dtype):
    wl = _wl("sf32q", 2, 17, 20, 2, 32, dtype, seed=5, state_std=0.3, separate_q=True)
    _both(wl, record=True)
    _both(wl, flags=srnl.FLAG_HARD_CAP | srnl.FLAG_FREEZE_KV)


@pytest.mark.parametrize("d,heads,flags", [(16, 2, 0), (32, 2, srnl.FLAG_READ_BEFORE),
                                           (64, 1, 0), (8, 3, srnl.FLAG_NO_CLAMP)])
def test_through_workspace_matches_two_calls(d, heads, flags):
    # no windowed d = 32 adjoint: dy_routes are written to the workspace
    _both(_wl(f"sfw{d}", 2, 9, 11, heads, d, "f32", seed=d, state_std=0.3), 15, flags)


def test_one_call_against_oracle():
    wl = _wl("sfo", 1, 6, 20, 2, 32, "f32", seed=9, state_std=0.3)
    dout, (dx, _, dst, dsc) = _both(wl)
    gx, _, gst, gsc = G.grads(wl.x, wl.states, wl.scales, wl.heads, wl.d, 15, None,
                              dy=np.zeros((4, wl.B, wl.N, wl.C), np.float32),
                              dfused=dout.cpu().numpy(), alpha_max=wl.alpha_max, eps=wl.eps,
                              chunk_row=wl.chunk_row, chunk_col=wl.chunk_col)
    for got, ref in ((dx, gx), (dst, gst), (dsc, gsc)):
        got = got.cpu().numpy()
        assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max()


def test_errors_and_empty_grid():
    wl = _wl("sfe", 1, 4, 5, 2, 32, "f32", seed=2)
    x = torch.from_numpy(wl.x).to(DEV)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    p = srnl.make_params(st, x, None, alpha_max=wl.alpha_max, eps=wl.eps)
    L = srnl.lib()
    import ctypes
    need = L.srnl_scan_fuse_bwd_workspace_bytes(1, 4, 5, 64, 2, 32, 15, ctypes.byref(p))
    assert need > 0
    y = srnl.scan_fwd(x, st, 2, 32, 15, None, alpha_max=wl.alpha_max, eps=wl.eps)
    dout = torch.ones((1, 4, 5, 64), device=DEV)
    out = [torch.empty((1, 4, 5, 64), device=DEV), torch.empty((4, 2, 3 * 32 * 32 + 64), device=DEV),
           torch.empty((4, 64), device=DEV)]
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    s = L.srnl_scan_fuse_bwd(x.data_ptr(), 1, 4, 5, 64, 2, 32, 15, ctypes.byref(p), y.data_ptr(),
                             sc.data_ptr(), dout.data_ptr(), ws.data_ptr(), need - 1,
                             out[0].data_ptr(), None, out[1].data_ptr(), out[2].data_ptr())
    assert s == srnl.SRNL_ERR_WORKSPACE
    s = L.srnl_scan_fuse_bwd(x.data_ptr(), 1, 4, 5, 64, 2, 32, 15, ctypes.byref(p), y.data_ptr(),
                             sc.data_ptr(), None, ws.data_ptr(), need,
                             out[0].data_ptr(), None, out[1].data_ptr(), out[2].data_ptr())
    assert s == srnl.SRNL_ERR_PTR
    assert L.srnl_scan_fuse_bwd_workspace_bytes(0, 4, 5, 64, 2, 32, 15, ctypes.byref(p)) == 0
    s = L.srnl_scan_fuse_bwd(x.data_ptr(), 0, 4, 5, 64, 2, 32, 15, ctypes.byref(p), None, None,
                             None, None, 0, None, None, None, None)
    assert s == srnl.SRNL_OK
