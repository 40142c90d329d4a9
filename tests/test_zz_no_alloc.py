"""srnl_fuse_bwd_noalloc (through the C ABI) against srnl_fuse_bwd: the
variant for callers that cannot allocate keeps its partial sums in the
library's own device array. Two calls in a row, the second on a smaller
input (the array keeps the first call's contents), must each give bitwise
the results of srnl_fuse_bwd with a caller workspace."""
import ctypes

import numpy as np
import pytest
import torch

from self_referential_memory_amd import srnl, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, H, W, C, mask, seed):
    R = bin(mask).count("1")
    rng = np.random.default_rng(seed)
    y = torch.from_numpy(rng.standard_normal((R, B, H * W, C)).astype(np.float32)).to(DEV)
    dout = torch.from_numpy(rng.standard_normal((B, H, W, C)).astype(np.float32)).to(DEV)
    sc = torch.from_numpy(synth.scales(seed, C)).to(DEV)
    return y, dout, sc


def _ref(y, dout, sc, B, H, W, C, mask):
    return srnl.fuse_bwd(dout, y, B, H, W, C, mask, sc)


def _noalloc(y, dout, sc, B, H, W, C, mask):
    L = srnl.lib()
    dyr = torch.empty_like(y)
    dsc = torch.empty((4, C), dtype=torch.float32, device=DEV)
    rc = L.srnl_fuse_bwd_noalloc(dout.data_ptr(), y.data_ptr(), B, H, W, C, mask,
                                 sc.data_ptr(), dyr.data_ptr(), dsc.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == srnl.SRNL_OK, L.srnl_last_error().decode()
    return dyr, dsc


def test_fuse_bwd_noalloc_matches_fuse_bwd_on_two_calls():
    # first a 56 x 56 map of 16 items (0.8 MB of partial sums), then a small
    # ragged one with two routes and fewer channels
    for (B, H, W, C, mask, seed) in ((16, 56, 56, 64, 15, 1), (2, 9, 11, 32, 5, 2)):
        print(f"[gpu] fuse_bwd_noalloc B={B} {H}x{W} C={C} mask={mask}", flush=True)
        y, dout, sc = _case(B, H, W, C, mask, seed)
        dyr, dsc = _noalloc(y, dout, sc, B, H, W, C, mask)
        ref_dyr, ref_dsc = _ref(y, dout, sc, B, H, W, C, mask)
        torch.cuda.synchronize()
        assert torch.equal(dyr, ref_dyr)
        assert torch.equal(dsc, ref_dsc)


def test_fuse_bwd_noalloc_rejects_sizes_beyond_its_scratch():
    L = srnl.lib()
    # 4 routes x ceil(700 * 56 * 56 / 256) blocks x 64 channels x 4 bytes > 8 MiB
    rc = L.srnl_fuse_bwd_noalloc(None, None, 700, 56, 56, 64, 15, None, None, None, None)
    assert rc == srnl.SRNL_ERR_WORKSPACE
    assert "scratch" in L.srnl_last_error().decode()
