"""GPU parity of srnl_block_fwd (one residual block around the operator)
against the float64 block oracle, element by element.

The block's workspace holds every intermediate (u, q, the fused operator
output s, the route outputs y), so each stage is compared as well as the
output. Bars: 1e-5 of the largest magnitude for u and q (layer norm and one
projection in fp32 with exact bf16-split products), 1e-4 for y, s and an
fp32 output (the operator's bar), and for a bf16 output one bf16 rounding
(2^-8 of each element) plus 1e-5 of the largest magnitude.
"""
import numpy as np
import pytest
import torch

from oracle import block as OB
from self_referential_memory_amd import srnl, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev_weights(bw):
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)
    return dict(ln1_w=t(bw.ln1_w), ln1_b=t(bw.ln1_b), wq=t(bw.wq, torch.bfloat16),
                dw_w=t(bw.dw_w), dw_b=t(bw.dw_b), ln2_w=t(bw.ln2_w), ln2_b=t(bw.ln2_b),
                w1=t(bw.w1, torch.bfloat16), b1=t(bw.b1), w2=t(bw.w2, torch.bfloat16),
                b2=t(bw.b2))


def _rel(g, o):
    m = np.abs(o).max()
    return float(np.abs(g - o).max() / m) if m > 0 else float(np.abs(g).max())


def run_block(wl, bw, route_mask=15, flags=0, items=None):
    """Run the block on the GPU; compare with the oracle on batch items
    ``items`` (all when None)."""
    print(f"[block] {wl.name} B={wl.B} {wl.H}x{wl.W} C={wl.C} heads={wl.heads} d={wl.d} "
          f"F={bw.F} dtype={wl.dtype} mask={route_mask} flags={flags}", flush=True)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    dw = _dev_weights(bw)
    w = srnl.block_weights(dw, sc, bw.ln_eps)
    nbytes = srnl.lib().srnl_block_workspace_bytes(B, H, W, C, route_mask)
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device=DEV)
    out = srnl.block_fwd(x, st, w, wl.heads, wl.d, route_mask, workspace=ws,
                         alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
                         chunk_col=wl.chunk_col, flags=flags)
    torch.cuda.synchronize()
    plane = (B * H * W * C + 63) // 64 * 64
    R = bin(route_mask).count("1")
    wsn = ws.cpu().numpy()
    gu = wsn[:B * H * W * C].reshape(B, H, W, C)
    gq = wsn[plane:plane + B * H * W * C].reshape(B, H, W, C)
    gs = wsn[2 * plane:2 * plane + B * H * W * C].reshape(B, H, W, C)
    gy = wsn[3 * plane:3 * plane + R * B * H * W * C].reshape(R, B, H * W, C)
    gout = out.float().cpu().numpy()
    sel = list(range(B)) if items is None else list(items)
    cap = dict(cap_mode=0 if not flags & 3 else (1 if flags & 1 else 2),
               clamp=not flags & srnl.FLAG_NO_CLAMP,
               fixed_alpha=bool(flags & srnl.FLAG_FIXED_ALPHA),
               readout_before=bool(flags & srnl.FLAG_READ_BEFORE),
               freeze_kv=bool(flags & srnl.FLAG_FREEZE_KV))
    p = OB.block_forward(wl.x[sel], wl.states, wl.scales, bw, wl.heads, wl.d, route_mask,
                         threads=8, parts=True, alpha_max=wl.alpha_max, eps=wl.eps,
                         chunk_row=wl.chunk_row, chunk_col=wl.chunk_col, **cap)
    assert _rel(gu[sel], p["u"]) <= 1e-5, "u"
    assert _rel(gq[sel], p["q"]) <= 1e-5, "q"
    for r in range(R):
        assert _rel(gy[r][sel], p["y"][r]) <= 1e-4, f"y slot {r}"
    assert _rel(gs[sel], p["s"]) <= 1e-4, "s"
    o = p["out"]
    g = gout[sel]
    if wl.dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(o) + 1e-5 * np.abs(o).max()
        assert (np.abs(g - o) <= bound).all(), float((np.abs(g - o) - bound).max())
    else:
        assert _rel(g, o) <= 1e-4, "out"
    return gout, p


def test_block_small_fp32():
    wl = synth.make("blk_small", 2, 8, 11, 64, 2, 32, "f32", 31, state_std=0.5)
    run_block(wl, synth.block_weights(31, 64, 256))


def test_block_bf16_wide_and_ragged():
    # 5 x 7 = 35 tokens per item: the last 64-token tile of the kernels is ragged
    wl = synth.make("blk_bf16", 3, 5, 7, 128, 4, 32, "bf16", 32, state_std=0.5)
    run_block(wl, synth.block_weights(32, 128, 512))


@pytest.mark.parametrize("C,heads,d,F_", [(32, 2, 16, 64), (192, 3, 64, 768), (256, 8, 32, 1024),
                                          (64, 2, 32, 96)])
def test_block_channel_widths(C, heads, d, F_):
    wl = synth.make(f"blk_c{C}", 2, 6, 9, C, heads, d, "f32", 33 + C, state_std=0.5)
    run_block(wl, synth.block_weights(33 + C, C, F_))


@pytest.mark.parametrize("dtype,B,H,W_,F_", [("f32", 2, 5, 7, 256), ("bf16", 2, 7, 7, 2048)])
def test_block_stage4_width(dtype, B, H, W_, F_):
    """C = 512 (16 heads of d = 32), the hierarchical model's last stage: the
    wide kernels. 5 x 7 leaves a ragged last block of tokens; 7 x 7 with
    F = 4C is the stage-4 map."""
    wl = synth.make(f"blk_c512_{dtype}", B, H, W_, 512, 16, 32, dtype, 36, state_std=0.5)
    run_block(wl, synth.block_weights(36, 512, F_))


def test_block_variants_and_route_subset():
    wl = synth.make("blk_var", 2, 7, 10, 64, 2, 32, "f32", 34, state_std=2.0, outlier_frac=0.05,
                    chunk_row=4, chunk_col=3)
    run_block(wl, synth.block_weights(34, 64, 256), route_mask=5,
              flags=srnl.FLAG_HARD_CAP | srnl.FLAG_FREEZE_KV)


def test_block_hier56_sampled_items():
    """The full 56x56 stage-1 shape (B = 64, C = 64, 2 heads x 32, bf16) in
    the launch configuration the benchmark times; batch items are
    independent, so the oracle checks the first and the last item."""
    wl = synth.hier56()
    run_block(wl, synth.block_weights(2, 64, 256), items=[0, 63])


def test_block_rejects_separate_queries_and_misaligned_weights():
    wl = synth.make("blk_err", 1, 4, 4, 64, 2, 32, "f32", 35)
    x = torch.from_numpy(wl.x).to(DEV)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    dw = _dev_weights(synth.block_weights(35, 64, 256))
    w = srnl.block_weights(dw, sc)
    with pytest.raises(srnl.SrnlError) as e:
        srnl.block_fwd(x, st, w, 2, 32, 15, params=srnl.make_params(st, x, x.clone()))
    assert e.value.status == srnl.SRNL_ERR_ARG
    big = torch.zeros(64 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    dw["wq"] = big[4:4 + 64 * 64].view(64, 64)        # 8-byte offset
    w = srnl.block_weights(dw, sc)
    with pytest.raises(srnl.SrnlError) as e:
        srnl.block_fwd(x, st, w, 2, 32, 15)
    assert e.value.status == srnl.SRNL_ERR_PTR
