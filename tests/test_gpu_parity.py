"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded input bytes.

Bars (max relative error = max |gpu - oracle| / max |oracle|, per route slot
and for the fused output):
  * fp32 per-route scan outputs: 1e-4, for fp32 and for bf16 inputs (both
    sides read the same bf16 bytes, so only fp32 arithmetic separates them);
  * fused output in fp32: 1e-4; fused output stored as bf16: 2e-2;
  * additionally, per chunk and batch item, on that chunk's own output scale:
    max |gpu - oracle| <= max(1e-4, 10 e32), where e32 is the largest error
    (same measure) of four fp32 evaluations of that chunk: the oracle's fp32
    build (every state, product and sum in IEEE single precision) on the
    given inputs, and on three copies of the inputs and states whose elements
    are multiplied by 1 +- 2^-24 (seeded random signs). This checks the late
    chunks of long scans, where the untrained memories have contracted by
    many orders of magnitude, on their own scale. Single chunks can be so
    ill-conditioned that no fp32 evaluation meets 1e-4 on them (the fp32 build
    reaches 4.5e-4 on a chunk of the adversarial inputs and 2.3e-3 on one of a
    56x56 grid with states of std 0.5, and one fp32 evaluation alone can be
    20x luckier than another on the same chunk; tests/test_oracle_fp32.py
    pins this); the bar follows that measured conditioning, chunk by chunk, and is
    1e-4 wherever fp32 evaluation is accurate to 1e-5. Chunks whose
    double-precision output is below 1e-20 are left out (fp32 underflows
    there);
  * route gather/restore indexing: bit-exact.
Full-size workloads run on the GPU in full; the oracle checks every batch
item of the five workloads and sampled items of the larger launches (chains
are independent across the batch, so a sample is exact).
"""
import ctypes
import itertools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from self_referential_memory_amd import srnl, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL32 = 1e-4
CHUNK_FACTOR = 10.0
FP32_REALISATIONS = 4
TOL_BF16_OUT = 2e-2
CHUNK_FLOOR = 1e-20
THREADS = max(1, min(16, os.cpu_count() or 1))


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV).to(dtype) if dtype != torch.float32 else t.to(DEV)


def gpu_forward(wl, route_mask=None, flags=0, out_dtype=None):
    rm = wl.route_mask if route_mask is None else route_mask
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    print(f"[gpu] {wl.name} B={wl.B} {wl.H}x{wl.W} C={wl.C} {wl.heads}x{wl.d} "
          f"mask={rm} flags={flags} chunks=({wl.chunk_row},{wl.chunk_col})", flush=True)
    x = _dev(wl.x, dt)
    q = None if wl.q is None else _dev(wl.q, dt)
    st = _dev(wl.states, torch.float32)
    sc = _dev(wl.scales, torch.float32)
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, rm, q, alpha_max=wl.alpha_max, eps=wl.eps,
                      chunk_row=wl.chunk_row, chunk_col=wl.chunk_col, flags=flags)
    out = srnl.fuse(y, wl.B, wl.H, wl.W, wl.C, rm, sc,
                    out_dtype=dt if out_dtype is None else out_dtype)
    torch.cuda.synchronize()
    return y.double().cpu().numpy(), out.double().cpu().numpy()


_CAP = {0: oracle.CAP_SOFT, srnl.FLAG_HARD_CAP: oracle.CAP_HARD, srnl.FLAG_NO_CAP: oracle.CAP_OFF}


def oracle_forward(wl, bs=None, route_mask=None, flags=0, threads=THREADS, fp32=False):
    """Oracle on batch items `bs` (all if None), one thread per (b, route).
    With fp32, also FP32_REALISATIONS fp32 evaluations of the same items (the
    fp32 build on the inputs and on perturbed copies: the conditioning of each
    chunk): returns y, fused, [y32, ...]."""
    rm = wl.route_mask if route_mask is None else route_mask
    bs = list(range(wl.B)) if bs is None else list(bs)
    routes = [r for r in range(4) if (rm >> r) & 1]
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps, chunk_row=wl.chunk_row,
              chunk_col=wl.chunk_col, cap_mode=_CAP[flags & 0x3],
              clamp=not (flags & srnl.FLAG_NO_CLAMP),
              fixed_alpha=bool(flags & srnl.FLAG_FIXED_ALPHA),
              readout_before=bool(flags & srnl.FLAG_READ_BEFORE),
              freeze_kv=bool(flags & srnl.FLAG_FREEZE_KV))
    inputs = {"f64": (wl.x, wl.q, wl.states)}
    if fp32:
        inputs[0] = (wl.x, wl.q, wl.states)
        for k in range(1, FP32_REALISATIONS):
            inputs[k] = (oracle.perturbed(wl.x, 3 * k), oracle.perturbed(wl.q, 3 * k + 1),
                         oracle.perturbed(wl.states, 3 * k + 2))

    def job(brk):
        b, r, key = brk
        x, q, st = inputs[key]
        qb = None if q is None else q[b:b + 1]
        return oracle.scan(x[b:b + 1], st, wl.heads, wl.d, 1 << r, qb,
                           precision="f64" if key == "f64" else "f32", **kw)[0, 0]

    jobs = list(itertools.product(bs, routes, list(inputs)))
    with ThreadPoolExecutor(max(1, min(threads, len(jobs)))) as ex:
        res = list(ex.map(job, jobs))
    ys = {k: np.zeros((len(routes), len(bs), wl.N, wl.C)) for k in inputs}
    for (b, r, key), yr in zip(jobs, res):
        ys[key][routes.index(r), bs.index(b)] = yr
    fused = oracle.fuse(ys["f64"], len(bs), wl.H, wl.W, wl.C, rm, wl.scales)
    if fp32:
        return ys["f64"], fused, [ys[k] for k in range(FP32_REALISATIONS)]
    return ys["f64"], fused


def rel(g, o):
    m = np.abs(o).max()
    return np.abs(g - o).max() / m if m > 0 else np.abs(g).max()


def chunk_errors(g, o, L):
    """Per (chunk, batch item): max |g - o| over the chunk's tokens relative to
    max |o| there, and max |o|. g, o: [B,N,C]; returns two [chunks, B] arrays."""
    N = o.shape[1]
    errs, scales = [], []
    for c0 in range(0, N, L):
        m = np.abs(o[:, c0:c0 + L]).max(axis=(1, 2))
        e = np.abs(g[:, c0:c0 + L] - o[:, c0:c0 + L]).max(axis=(1, 2))
        scales.append(m)
        errs.append(np.where(m > 0, e / np.where(m > 0, m, 1.0), e))
    return np.array(errs), np.array(scales)


def check_chunks(g, o, reals, L, what):
    """Every chunk above CHUNK_FLOOR within max(TOL32, CHUNK_FACTOR e32) of the
    oracle, e32 being the largest error of the fp32 evaluations `reals` on the
    same chunk. Returns the number of chunks checked."""
    eg, m = chunk_errors(g, o, L)
    e32 = np.max([chunk_errors(y, o, L)[0] for y in reals], axis=0)
    live = m > CHUNK_FLOOR
    bar = np.maximum(TOL32, CHUNK_FACTOR * e32)
    bad = live & (eg > bar)
    if bad.any():
        c, b = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: chunk {c} of item {b}: error {eg[c, b]:.3e} > bar "
                             f"{bar[c, b]:.3e} (fp32 build {e32[c, b]:.3e}); "
                             f"{int(bad.sum())} chunks over")
    return int(live.sum())


def check(wl, bs=None, route_mask=None, flags=0, out_dtype=None):
    yg, fg = gpu_forward(wl, route_mask, flags, out_dtype)
    yo, fo, y32 = oracle_forward(wl, bs, route_mask, flags, fp32=True)
    if bs is not None:
        yg, fg = yg[:, list(bs)], fg[list(bs)]
    assert np.isfinite(yg).all()
    rm = wl.route_mask if route_mask is None else route_mask
    routes = [r for r in range(4) if (rm >> r) & 1]
    for s, r in enumerate(routes):
        e = rel(yg[s], yo[s])
        assert e <= TOL32, (wl.name, "slot", s, e)
        L = min(oracle.chunk_len(r, wl.H, wl.W, wl.chunk_row, wl.chunk_col), wl.N)
        check_chunks(yg[s], yo[s], [y[s] for y in y32], L, f"{wl.name} slot {s}")
    bf = (wl.dtype == "bf16") if out_dtype is None else (out_dtype == torch.bfloat16)
    e = rel(fg, fo)
    assert e <= (TOL_BF16_OUT if bf else TOL32), (wl.name, "fused", e)
    return yg, yo


# ----------------------------------------------------------- init / gather

@pytest.mark.parametrize("heads,d,seed,std", [(1, 16, 0, 0.02), (3, 64, 1, 0.02),
                                              (2, 32, 2, 0.5), (5, 4, 99, 1.0)])
def test_init_states_matches_generator(heads, d, seed, std):
    g = srnl.init_states(heads, d, seed, std).cpu().numpy()
    ref = synth.states(seed, heads, d, std)
    assert g.shape == ref.shape
    gi, ri = g.view(np.int32).astype(np.int64), ref.view(np.int32).astype(np.int64)
    assert np.abs(gi - ri).max() <= 1          # within one fp32 ulp
    assert (gi == ri).mean() > 0.999            # and bit-exact almost everywhere


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H,W,C,mask", [(2, 5, 7, 8, 15), (1, 1, 9, 4, 15), (3, 6, 1, 12, 5),
                                          (2, 56, 56, 64, 15), (1, 200, 304, 64, 10)])
def test_route_gather_bit_exact(dtype, B, H, W, C, mask):
    x = _dev(synth.normals(7, 1, B * H * W * C).reshape(B, H, W, C), dtype)
    g = srnl.route_gather(x, mask)
    routes = [r for r in range(4) if (mask >> r) & 1]
    xf = x.reshape(B, H * W, C)
    for s, r in enumerate(routes):
        cells = [oracle.route_index(r, H, W, t) for t in range(H * W)]
        idx = torch.tensor([i * W + j for i, j in cells], device=DEV)
        assert torch.equal(g[s], xf[:, idx])


@pytest.mark.parametrize("dtype,offset", [(torch.bfloat16, 1), (torch.bfloat16, 2),
                                          (torch.bfloat16, 4), (torch.float32, 1),
                                          (torch.float32, 2)])
@pytest.mark.parametrize("C", [4, 12, 2052])
def test_route_gather_unaligned_views_and_wide_rows(dtype, offset, C):
    """Views that start 2, 4 or 8 bytes past an aligned address take the
    narrower copy widths; rows wider than 256 vectors loop over channels."""
    B, H, W, mask = 2, 3, 5, 15
    base = _dev(synth.normals(8, 1, B * H * W * C + offset), dtype)
    x = base[offset:].view(B, H, W, C)
    g = srnl.route_gather(x, mask)
    xf = x.reshape(B, H * W, C)
    for r in range(4):
        cells = [oracle.route_index(r, H, W, t) for t in range(H * W)]
        idx = torch.tensor([i * W + j for i, j in cells], device=DEV)
        assert torch.equal(g[r], xf[:, idx])


def test_fuse_wide_rows():
    """C = 1028: more 4-channel vectors per token (257) than a block holds."""
    B, H, W, C, mask = 2, 3, 2, 1028, 15
    y = synth.normals(4, 1, 4 * B * H * W * C).reshape(4, B, H * W, C).astype(np.float32)
    sc = synth.scales(4, C)
    out = srnl.fuse(_dev(y, torch.float32), B, H, W, C, mask,
                    _dev(sc, torch.float32)).double().cpu().numpy()
    exp = oracle.fuse(y.astype(np.float64), B, H, W, C, mask, sc)
    assert np.abs(out - exp).max() <= 1e-6 * np.abs(exp).max()


@pytest.mark.parametrize("mask", [1, 2, 4, 8, 6, 15])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fuse_matches_oracle(mask, out_dtype):
    B, H, W, C = 2, 7, 9, 16
    R = bin(mask).count("1")
    y = synth.normals(3, 1, R * B * H * W * C).reshape(R, B, H * W, C).astype(np.float32)
    sc = synth.scales(3, C)
    out = srnl.fuse(_dev(y, torch.float32), B, H, W, C, mask, _dev(sc, torch.float32),
                    out_dtype=out_dtype).double().cpu().numpy()
    exp = oracle.fuse(y.astype(np.float64), B, H, W, C, mask, sc)
    if out_dtype == torch.float32:
        assert np.abs(out - exp).max() <= 1e-6 * np.abs(exp).max()
    else:
        assert rel(out, exp) <= TOL_BF16_OUT
        assert np.all(np.abs(out - exp) <= np.abs(exp) * 2 ** -8 + 1e-6)


@pytest.mark.parametrize("r", [0, 1, 2, 3])
def test_fuse_single_route_unit_scale_is_exact_restore(r):
    B, H, W, C = 2, 6, 11, 8
    y = synth.normals(5, 1, B * H * W * C).reshape(1, B, H * W, C).astype(np.float32)
    out = srnl.fuse(_dev(y, torch.float32), B, H, W, C, 1 << r,
                    torch.ones(4, C, device=DEV)).cpu().numpy()
    cells = [oracle.route_index(r, H, W, t) for t in range(H * W)]
    exp = np.zeros((B, H, W, C), np.float32)
    for t, (i, j) in enumerate(cells):
        exp[:, i, j] = y[0, :, t]
    assert np.array_equal(out, exp)


# ----------------------------------------------------------- the five workloads

def test_tiny_config_full():
    check(synth.tiny())


def test_plain14_full_batch():
    check(synth.plain14())


def test_hier56_full_batch():
    check(synth.hier56())


def test_hier56_launch_live_states_every_chunk():
    """The benchmark's launch (B = 64, 56 x 56, C = 64, 2 heads of d = 32,
    bf16, AR(1) rows: the 64-token sub-block on four waves) on states that
    keep every chunk alive: retention fixed at 0.999 and states of std 1.
    With the benchmark's own states the memories contract by ~1e-9 per chunk
    and the outputs leave fp32's range after a few chunks; here the smallest
    chunk scale stays near 1, so every one of the 56 chunks of every route
    and batch item is checked on its own scale."""
    wl = synth.hier56_live()
    yg, fg = gpu_forward(wl, flags=srnl.FLAG_FIXED_ALPHA)
    yo, fo, y32 = oracle_forward(wl, flags=srnl.FLAG_FIXED_ALPHA, fp32=True)
    assert np.isfinite(yg).all()
    for s in range(4):
        assert rel(yg[s], yo[s]) <= TOL32, (s, rel(yg[s], yo[s]))
        n = check_chunks(yg[s], yo[s], [y[s] for y in y32], 56, f"live slot {s}")
        assert n == 56 * wl.B          # every chunk of every item is live
    assert rel(fg, fo) <= TOL_BF16_OUT


@pytest.mark.parametrize("stage", [0, 1, 2, 3])
def test_hier_sweep_stage(stage):
    check(synth.hier_sweep()[stage])


def test_dense200x304_full():
    check(synth.dense200x304())


# ----------------------------------------------------------- stress and edges

def test_single_chunk_long_scan_stays_alive():
    wl = synth.hier56(B=2)
    wl.chunk_row = wl.chunk_col = wl.N     # one chunk: memory stays O(1) for 3136 tokens
    yg, yo = check(wl)
    assert np.abs(yo[:, :, -100:]).max() > 1e-4


def test_fixed_retention_near_one_stays_alive():
    wl = synth.make("fixed999", 2, 28, 28, 64, 2, 32, "bf16", 12, alpha_max=0.999)
    yg, yo = check(wl, flags=srnl.FLAG_FIXED_ALPHA)
    assert np.abs(yo[:, :, -10:]).max() > 1e-4


@pytest.mark.parametrize("cr,cc", [(13, 9), (1, 1), (3, 200), (64, 64), (1000, 7)])
def test_chunk_overrides_with_ragged_tails(cr, cc):
    wl = synth.make("ragged", 2, 14, 20, 64, 4, 16, "f32", 13, state_std=0.3,
                    chunk_row=cr, chunk_col=cc)
    check(wl)


@pytest.mark.parametrize("B,H,W", [(1, 1, 1), (1, 1, 37), (2, 37, 1), (1, 2, 2), (3, 5, 64)])
def test_degenerate_grids(B, H, W):
    check(synth.make("degenerate", B, H, W, 32, 1, 32, "f32", 14, state_std=0.3))


@pytest.mark.parametrize("d,heads", [(4, 3), (8, 2), (16, 4), (32, 2), (64, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_head_dim(d, heads, dtype):
    check(synth.make("headdim", 2, 9, 13, heads * d, heads, d, dtype, 15, state_std=0.3))


@pytest.mark.parametrize("mask", [1, 2, 4, 8, 3, 12, 5, 10, 7, 14])
def test_route_subsets(mask):
    check(synth.make("mask", 2, 8, 11, 32, 2, 16, "f32", 16, state_std=0.3), route_mask=mask)


@pytest.mark.parametrize("flags", [0, srnl.FLAG_HARD_CAP, srnl.FLAG_NO_CAP, srnl.FLAG_NO_CLAMP,
                                   srnl.FLAG_FIXED_ALPHA, srnl.FLAG_READ_BEFORE,
                                   srnl.FLAG_HARD_CAP | srnl.FLAG_NO_CLAMP, srnl.FLAG_FREEZE_KV])
def test_variants_on_adversarial_inputs(flags):
    # large state spread and x50 outlier tokens: the cap and the clamp bind.
    # Without the cap these inputs are expansive (memory norms grow ~6e15x
    # over the boundary's), so rounding differences grow without bound and
    # the no-cap ablation is checked on milder states (std 0.3, growth 3.5x).
    if flags & srnl.FLAG_NO_CAP:
        wl = synth.make("nocap", 2, 12, 10, 64, 2, 32, "f32", 17, state_std=0.3)
    else:
        wl = synth.make("adv", 2, 12, 10, 64, 2, 32, "f32", 17, state_std=3.0, outlier_frac=0.05)
    check(wl, flags=flags)


def test_clamp_binds_in_adversarial_parity_case():
    wl = synth.make("adv", 2, 12, 10, 64, 2, 32, "f32", 17, state_std=3.0, outlier_frac=0.05)
    _, tr = oracle.scan(wl.x, wl.states, 2, 32, 15, trace=True)
    assert (tr[..., 13] < tr[..., 12]).mean() > 0.001


# The scan kernel picks its sub-block from the longest chunk: at d = 32, 16
# or 32 tokens (on two waves) for chunks that fit, else 64 tokens, or 128 on
# eight waves when there are at most 256 chains; at d = 64, 16 or 32 tokens.
# Each configuration runs on large states with x50 outlier tokens, where the
# clamp binds on 1-5 % of the tokens, with variant flags, both input dtypes
# and separate queries. The states are chosen so that no chunk of a grid
# moves by more than 2.2e-4 of its scale when the inputs are perturbed at the
# fp32 rounding level in exact arithmetic (std 3 puts a chunk of the 14x14
# d = 64 grid at 1.3e-3, beyond the per-chunk bar for any fp32 evaluation).
SUB_BLOCK_GRIDS = [
    # name, B, H, W, d, heads, chunk_row, chunk_col, state_std, outlier_frac
    ("sb16_d32", 2, 12, 10, 32, 2, 0, 0, 2.0, 0.05),
    ("sb32_d32", 2, 20, 28, 32, 2, 0, 0, 2.0, 0.05),
    ("sb64_d32", 1, 10, 55, 32, 2, 45, 0, 2.0, 0.05),    # 45-token row chunks, ragged tail
    ("sb128_d32", 1, 6, 150, 32, 2, 0, 0, 2.0, 0.05),   # 8 chains; 150 = 128 + 22
    ("sb64x2_d32", 40, 3, 100, 32, 2, 0, 0, 0.5, 0.0),  # 320 chains; 100 = 64 + 36
    ("sb16_d64", 2, 14, 14, 64, 1, 0, 0, 2.0, 0.05),
    ("sb32_d64", 1, 24, 20, 64, 1, 0, 0, 2.0, 0.05),
]
SUB_BLOCK_VARIANTS = [
    (0, "bf16", False),
    (srnl.FLAG_READ_BEFORE, "f32", True),
    (srnl.FLAG_HARD_CAP | srnl.FLAG_NO_CLAMP, "f32", False),
    (srnl.FLAG_FIXED_ALPHA, "bf16", True),
    (srnl.FLAG_FREEZE_KV, "bf16", False),
]


@pytest.mark.parametrize("grid", SUB_BLOCK_GRIDS, ids=[g[0] for g in SUB_BLOCK_GRIDS])
@pytest.mark.parametrize("variant", SUB_BLOCK_VARIANTS, ids=["plain", "before_q", "hardcap_noclamp",
                                                              "fixedalpha_q", "freeze"])
def test_sub_block_configurations(grid, variant):
    name, B, H, W, d, heads, cr, cc, std, outl = grid
    flags, dtype, q = variant
    wl = synth.make(name, B, H, W, heads * d, heads, d, dtype, 21, state_std=std,
                    outlier_frac=outl, separate_q=q, chunk_row=cr, chunk_col=cc)
    check(wl, flags=flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_separate_queries(dtype):
    check(synth.make("q", 2, 10, 12, 64, 2, 32, dtype, 18, state_std=0.3, separate_q=True))


def test_zero_input_closed_form_on_gpu():
    wl = synth.make("zero", 1, 4, 6, 32, 2, 16, "f32", 19, x_kind="zero", separate_q=True)
    yg, _ = gpu_forward(wl)
    H, W, d = 4, 6, 16
    for s, r in enumerate(range(4)):
        cells = [oracle.route_index(r, H, W, t) for t in range(H * W)]
        Q = np.stack([wl.q[0, i, j] for i, j in cells]).astype(np.float64)
        for h in range(2):
            Mc = wl.states[r, h, :d * d].reshape(d, d).astype(np.float64)
            f = 0.45 ** (np.arange(H * W) + 1)
            exp = f[:, None] * (Q[:, h * d:(h + 1) * d] @ Mc.T)
            got = yg[s, 0, :, h * d:(h + 1) * d]
            assert np.all(np.abs(got - exp) <= 1e-4 * np.abs(exp).max(axis=1, keepdims=True))


def test_fp32_output_of_bf16_input():
    check(synth.plain14(B=2), out_dtype=torch.float32)


# ----------------------------------------------------------- determinism, errors

def test_bitwise_deterministic_across_runs_and_streams():
    wl = synth.hier56(B=4)
    a, fa = gpu_forward(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b, fb = gpu_forward(wl)
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(fa, fb)


def test_host_pointer_is_rejected():
    x = torch.zeros(1, 2, 2, 8)
    st = torch.zeros(4, 2, 56, device=DEV)
    with pytest.raises(srnl.SrnlError) as ei:
        srnl.scan_fwd(x, st, 2, 4, 15, out=torch.empty(4, 1, 4, 8, device=DEV))
    assert ei.value.status == srnl.SRNL_ERR_PTR


def test_empty_batch_launches_nothing():
    x = torch.zeros(0, 3, 3, 8, device=DEV)
    st = torch.zeros(4, 2, 56, device=DEV)
    y = srnl.scan_fwd(x, st, 2, 4, 15)
    assert y.shape == (4, 0, 9, 8)


# ------------------------------------------------------------ standalone 1-D SRNL

def _seq(B, N, C, heads, d, seed, dtype="f32", separate_q=False):
    """Seeded [B][N][C] sequence, [heads][3d^2+2d] states and optional queries."""
    x = synth.normals(seed, 1, B * N * C).reshape(B, N, C).astype(np.float32)
    st = synth.states(seed, heads, d, 0.02)[0]          # [heads][3d^2+2d]
    q = synth.normals(seed, 5, B * N * C).reshape(B, N, C).astype(np.float32) if separate_q else None
    if dtype == "bf16":
        x = synth.round_bf16(x)[0]
        q = None if q is None else synth.round_bf16(q)[0]
    return x, st, q


def _scan_1d_fp32(x, st, heads, d, q=None, chunk=0):
    """FP32_REALISATIONS fp32 evaluations of the 1-D scan (the oracle's fp32
    build on the inputs and on perturbed copies)."""
    out = [oracle.scan_1d(x, st, heads, d, q, chunk=chunk, precision="f32")]
    for k in range(1, FP32_REALISATIONS):
        out.append(oracle.scan_1d(oracle.perturbed(x, 3 * k), oracle.perturbed(st, 3 * k + 2), heads, d,
                                  oracle.perturbed(q, 3 * k + 1), chunk=chunk, precision="f32"))
    return out


def _scan_1d_gpu(x, st, heads, d, q=None, dtype="f32", chunk=0):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"[gpu] scan_1d B={x.shape[0]} N={x.shape[1]} C={x.shape[2]} {heads}x{d} "
          f"{dtype} chunk={chunk} q={q is not None}", flush=True)
    xg = _dev(x, dt)
    qg = None if q is None else _dev(q, dt)
    y = srnl.scan_1d(xg, _dev(st, torch.float32), heads, d, qg, chunk=chunk)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 100])
def test_scan_1d_matches_oracle(d, dtype, chunk):
    """README operator shape: [2, 257, 64], default 64-token chunks (short final
    chunk of 1 token) and a 100-token override."""
    B, N, C = 2, 257, 64
    heads = C // d
    x, st, _ = _seq(B, N, C, heads, d, seed=40 + d, dtype=dtype)
    yg = _scan_1d_gpu(x, st, heads, d, dtype=dtype, chunk=chunk)
    yo = oracle.scan_1d(x, st, heads, d, chunk=chunk)
    y32 = _scan_1d_fp32(x, st, heads, d, chunk=chunk)
    assert np.isfinite(yg).all()
    assert rel(yg, yo) <= TOL32, rel(yg, yo)
    check_chunks(yg, yo, y32, chunk if chunk > 0 else 64, "1-D")


def test_scan_1d_bench_workload_sampled():
    """The 1-D benchmark workload in its launch configuration (256 sequences
    of 3136 tokens, 2 heads x d = 32, bf16, 64-token chunks); sequences are
    independent, so the oracle checks the first and the last."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                              "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    x, st, heads, d = bench.seq1d_workload()
    yg = _scan_1d_gpu(x, st, heads, d, dtype="bf16")
    sel = [0, x.shape[0] - 1]
    yo = oracle.scan_1d(x[sel], st, heads, d)
    y32 = _scan_1d_fp32(x[sel], st, heads, d)
    assert np.isfinite(yg).all()
    assert rel(yg[sel], yo) <= TOL32
    check_chunks(yg[sel], yo, y32, 64, "1-D bench workload")


@pytest.mark.parametrize("N", [1, 63, 64, 65, 1000])
def test_scan_1d_lengths(N):
    B, C, heads, d = 3, 64, 2, 32
    x, st, _ = _seq(B, N, C, heads, d, seed=N)
    yg = _scan_1d_gpu(x, st, heads, d)
    yo = oracle.scan_1d(x, st, heads, d)
    y32 = _scan_1d_fp32(x, st, heads, d)
    assert rel(yg, yo) <= TOL32
    check_chunks(yg, yo, y32, 64, "1-D lengths")


def test_scan_1d_separate_queries():
    B, N, C, heads, d = 2, 300, 64, 2, 32
    x, st, q = _seq(B, N, C, heads, d, seed=77, dtype="bf16", separate_q=True)
    yg = _scan_1d_gpu(x, st, heads, d, q=q, dtype="bf16")
    yo = oracle.scan_1d(x, st, heads, d, q=q)
    assert rel(yg, yo) <= TOL32


def test_scan_1d_equals_row_route_of_1xN_grid_bitwise():
    B, N, C, heads, d = 2, 200, 64, 2, 32
    x, st, _ = _seq(B, N, C, heads, d, seed=3, dtype="bf16")
    y1 = _scan_1d_gpu(x, st, heads, d, dtype="bf16")
    st4 = np.zeros((4,) + st.shape, np.float32)
    st4[0] = st
    xg = _dev(x.reshape(B, 1, N, C), torch.bfloat16)
    y2 = srnl.scan_fwd(xg, _dev(st4, torch.float32), heads, d, 1, chunk_row=64)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2.double().cpu().numpy()[0])


def test_scan_1d_query_dtype_must_match():
    x = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((1, 8, 64), dtype=torch.float32, device=DEV)
    st = torch.zeros((2, srnl_state(32)), dtype=torch.float32, device=DEV)
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_1d(x, st, 2, 32, q)
    assert e.value.status == srnl.SRNL_ERR_DTYPE


def srnl_state(d):
    return 3 * d * d + 2 * d


def test_misaligned_tensors_are_pointer_errors():
    """Every entry point but the gather moves 16-byte vectors and rejects a
    tensor that starts off a 16-byte boundary, before launching anything."""
    wl = synth.make("mis", 1, 4, 4, 64, 2, 32, "f32", 51)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    n = B * H * W * C
    base = torch.zeros(n + 4, dtype=torch.float32, device=DEV)
    good = torch.from_numpy(wl.x).to(DEV)
    bad = base[1:1 + n].view(B, H, W, C)            # 4 bytes past an aligned address
    bad.copy_(good)
    st = torch.from_numpy(wl.states).to(DEV)
    sc = torch.from_numpy(wl.scales).to(DEV)
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd(bad, st, wl.heads, wl.d, 15)
    assert e.value.status == srnl.SRNL_ERR_PTR
    y = srnl.scan_fwd(good, st, wl.heads, wl.d, 15)
    ybase = torch.zeros(y.numel() + 4, dtype=torch.float32, device=DEV)
    ybad = ybase[1:1 + y.numel()].view(y.shape)
    ybad.copy_(y)
    with pytest.raises(srnl.SrnlError) as e:
        srnl.fuse(ybad, B, H, W, C, 15, sc)
    assert e.value.status == srnl.SRNL_ERR_PTR
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_bwd(good, st, wl.heads, wl.d, ybad, 15)
    assert e.value.status == srnl.SRNL_ERR_PTR
    with pytest.raises(srnl.SrnlError) as e:
        srnl.fuse_bwd(bad, y, B, H, W, C, 15, sc)
    assert e.value.status == srnl.SRNL_ERR_PTR
    # the aligned calls still work
    srnl.fuse(y, B, H, W, C, 15, sc)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_check_finite_flag(dtype):
    """SRNL_FLAG_CHECK_FINITE: on finite inputs the outputs equal an unchecked
    call's bit for bit; a NaN or an Inf in x or in the separate queries makes
    the call return SRNL_ERR_NONFINITE with the number of such values."""
    print(f"[gpu] check_finite {dtype}", flush=True)
    wl = synth.make("fin", 2, 6, 7, 64, 2, 32, dtype, 61)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    st = torch.from_numpy(wl.states).to(DEV)
    flag = srnl.FLAG_CHECK_FINITE
    y0 = srnl.scan_fwd(x, st, wl.heads, wl.d, 15)
    y1 = srnl.scan_fwd(x, st, wl.heads, wl.d, 15, flags=flag)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)

    xb = x.clone()
    xb.view(-1)[5] = float("nan")
    xb.view(-1)[-1] = float("inf")
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd(xb, st, wl.heads, wl.d, 15, flags=flag)
    assert e.value.status == srnl.SRNL_ERR_NONFINITE
    assert "2 non-finite input values" in str(e.value)

    q = x.clone()
    q.view(-1)[100] = float("-inf")
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd(x, st, wl.heads, wl.d, 15, q=q, flags=flag)
    assert e.value.status == srnl.SRNL_ERR_NONFINITE
    assert "1 non-finite input values" in str(e.value)

    # a caller's workspace: too small is an error; a valid one is cleared on
    # every call, so a clean call after a failing one succeeds
    p = srnl.make_params(st, x, flags=flag)
    small = torch.empty(8, dtype=torch.uint8, device=DEV)
    p.workspace, p.workspace_bytes = small.data_ptr(), 8
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_fwd(x, st, wl.heads, wl.d, 15, params=p)
    assert e.value.status == srnl.SRNL_ERR_WORKSPACE
    nb = srnl.lib().srnl_scan_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                              ctypes.byref(p))
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    p.workspace, p.workspace_bytes = ws.data_ptr(), nb
    with pytest.raises(srnl.SrnlError):
        srnl.scan_fwd(xb, st, wl.heads, wl.d, 15, params=srnl.make_params(st, xb, flags=flag))
    pb = srnl.make_params(st, xb, flags=flag)
    pb.workspace, pb.workspace_bytes = ws.data_ptr(), nb
    with pytest.raises(srnl.SrnlError):
        srnl.scan_fwd(xb, st, wl.heads, wl.d, 15, params=pb)
    y2 = srnl.scan_fwd(x, st, wl.heads, wl.d, 15, params=p)
    torch.cuda.synchronize()
    assert torch.equal(y0, y2)


def test_check_finite_flag_1d():
    """srnl_scan_1d takes the same finite check as the 2-D scan."""
    print("[gpu] check_finite 1d", flush=True)
    x, st, _ = _seq(2, 100, 64, 2, 32, seed=62, dtype="bf16")
    xg = _dev(x, torch.bfloat16)
    stg = _dev(st, torch.float32)
    flag = srnl.FLAG_CHECK_FINITE
    y0 = srnl.scan_1d(xg, stg, 2, 32)
    y1 = srnl.scan_1d(xg, stg, 2, 32, flags=flag)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    xb = xg.clone()
    xb[1, 50, 7] = float("nan")
    with pytest.raises(srnl.SrnlError) as e:
        srnl.scan_1d(xb, stg, 2, 32, flags=flag)
    assert e.value.status == srnl.SRNL_ERR_NONFINITE
    assert "1 non-finite input values" in str(e.value)


@pytest.mark.parametrize("case", ["chunk100", "dense200x304"])
def test_forward_record_outputs_on_long_chunks(case):
    """The forward that keeps its record (SRNL_FLAG_RECORD) runs 64-token
    sub-blocks on every chunk longer than 32 tokens, where the plain forward
    may take 128-token ones: its outputs against the oracle on chunks that
    span several sub-blocks (100-token chunks; the dense map's 304- and
    200-token rows and columns, x50 outlier tokens)."""
    if case == "chunk100":
        wl = synth.make("rec100", 2, 12, 50, 64, 2, 32, "bf16", 41, state_std=0.5,
                        chunk_row=100, chunk_col=100)
    else:
        wl = synth.dense200x304()
    print(f"[gpu] record outputs {case}", flush=True)
    x = _dev(wl.x, torch.bfloat16)
    st = _dev(wl.states, torch.float32)
    y, rec = srnl.scan_fwd_record(x, st, wl.heads, wl.d, 15, alpha_max=wl.alpha_max,
                                  eps=wl.eps, chunk_row=wl.chunk_row, chunk_col=wl.chunk_col)
    torch.cuda.synchronize()
    assert rec is not None
    yg = y.double().cpu().numpy()
    yo, _, y32 = oracle_forward(wl, fp32=True)
    assert np.isfinite(yg).all()
    for s in range(4):
        assert rel(yg[s], yo[s]) <= TOL32, (s, rel(yg[s], yo[s]))
        L = min(oracle.chunk_len(s, wl.H, wl.W, wl.chunk_row, wl.chunk_col), wl.N)
        check_chunks(yg[s], yo[s], [y[s] for y in y32], L, f"record {case} slot {s}")
