"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/srnl.h declares, its host helpers agree with the oracle's route and
chunk definitions, and invalid arguments return their documented status
before any device work."""
import ctypes
import json
import os
import re

import pytest

import oracle
from self_referential_memory_amd import srnl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "srnl.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(srnl_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for f in ("srnl_scan_fwd", "srnl_fuse", "srnl_init_states", "srnl_route_gather"):
        assert f in names
    assert sorted(srnl.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = srnl.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


@pytest.mark.parametrize("H,W", [(1, 1), (2, 3), (14, 20), (7, 56), (200, 304)])
def test_route_index_matches_oracle(H, W):
    N = H * W
    ts = range(N) if N <= 4096 else list(range(0, N, 97)) + [N - 1]
    for r in range(4):
        for t in ts:
            assert srnl.route_index(r, H, W, t) == oracle.route_index(r, H, W, t)


def test_chunk_len_matches_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "chunking.json")))
    for case in g["cases"]:
        H, W, cr, cc = case["H"], case["W"], case["chunk_row"], case["chunk_col"]
        assert srnl.chunk_len(0, H, W, cr, cc) == case["row_chunk_len"]
        assert srnl.chunk_len(3, H, W, cr, cc) == case["col_chunk_len"]


def _scan(x=0, B=1, H=2, W=2, C=8, heads=2, d=4, mask=15, **kw):
    p = srnl.Params(None, None, kw.pop("in_dtype", 0), kw.pop("alpha_max", 0.9),
                    kw.pop("eps", 1e-6), kw.pop("chunk_row", 0), kw.pop("chunk_col", 0),
                    kw.pop("flags", 0), None)
    return srnl.lib().srnl_scan_fwd(x, B, H, W, C, heads, d, mask, ctypes.byref(p), None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=5, C=10), srnl.SRNL_ERR_ARG),          # head_dim not in {4,8,16,32,64}
    (dict(d=128, heads=1, C=128), srnl.SRNL_ERR_ARG),
    (dict(C=12), srnl.SRNL_ERR_ARG),                # C != heads * d
    (dict(heads=0, C=0), srnl.SRNL_ERR_ARG),
    (dict(mask=0), srnl.SRNL_ERR_ARG),
    (dict(mask=16), srnl.SRNL_ERR_ARG),
    (dict(B=-1), srnl.SRNL_ERR_ARG),
    (dict(H=-2), srnl.SRNL_ERR_ARG),
    (dict(alpha_max=1.0), srnl.SRNL_ERR_ARG),
    (dict(alpha_max=0.0), srnl.SRNL_ERR_ARG),
    (dict(alpha_max=float("nan")), srnl.SRNL_ERR_ARG),
    (dict(eps=0.0), srnl.SRNL_ERR_ARG),
    (dict(eps=float("inf")), srnl.SRNL_ERR_ARG),
    (dict(chunk_row=-1), srnl.SRNL_ERR_ARG),
    (dict(flags=0x100), srnl.SRNL_ERR_ARG),         # first bit above the known flags
    (dict(flags=0x200), srnl.SRNL_ERR_ARG),
    (dict(in_dtype=7), srnl.SRNL_ERR_DTYPE),
    (dict(B=1 << 30, H=1 << 15, W=1 << 15, heads=1, d=64, C=64), srnl.SRNL_ERR_ARG),  # overflow
    (dict(B=1, H=1 << 16, W=1 << 16, heads=1, d=64, C=64), srnl.SRNL_ERR_ARG),  # H*W > INT_MAX
])
def test_scan_argument_errors(kw, status):
    assert _scan(**kw) == status
    assert srnl.lib().srnl_last_error().decode() != ""


def test_null_params_is_pointer_error():
    assert srnl.lib().srnl_scan_fwd(0, 1, 2, 2, 8, 2, 4, 15, None, None) == srnl.SRNL_ERR_PTR


def test_empty_grid_is_a_no_op():
    # nothing to compute: valid, returns before touching any pointer
    assert _scan(B=0) == srnl.SRNL_OK
    assert _scan(H=0) == srnl.SRNL_OK
    assert srnl.lib().srnl_fuse(None, 0, 4, 4, 8, 15, None, 0, None, None) == srnl.SRNL_OK
    assert srnl.lib().srnl_route_gather(None, 3, 0, 4, 8, 15, 0, None, None) == srnl.SRNL_OK


def test_fuse_and_gather_argument_errors():
    L = srnl.lib()
    assert L.srnl_fuse(None, 1, 2, 2, 6, 15, None, 0, None, None) == srnl.SRNL_ERR_ARG  # C % 4
    assert L.srnl_fuse(None, 1, 2, 2, 8, 0, None, 0, None, None) == srnl.SRNL_ERR_ARG
    assert L.srnl_fuse(None, 1, 2, 2, 8, 15, None, 3, None, None) == srnl.SRNL_ERR_DTYPE
    assert L.srnl_route_gather(None, 1, 2, 2, 8, 31, 0, None, None) == srnl.SRNL_ERR_ARG
    assert L.srnl_route_gather(None, 1, 2, 2, 8, 15, 9, None, None) == srnl.SRNL_ERR_DTYPE
    assert L.srnl_init_states(None, 0, 4, 0, 0.02, None) == srnl.SRNL_ERR_ARG
    assert L.srnl_init_states(None, 1, 6, 0, 0.02, None) == srnl.SRNL_ERR_ARG
    assert L.srnl_init_states(None, 1, 4, 0, -1.0, None) == srnl.SRNL_ERR_ARG


def test_status_strings():
    L = srnl.lib()
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.srnl_status_string(s).decode() not in ("", "unknown status")


def test_scan_workspace_bytes():
    L = srnl.lib()

    def ws(flags, B=2, H=3, W=4, C=8, heads=2, d=4, mask=15):
        p = srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, flags, None)
        return L.srnl_scan_workspace_bytes(B, H, W, C, heads, d, mask, ctypes.byref(p))

    assert ws(0) == 0                               # no check: no workspace
    assert ws(srnl.FLAG_CHECK_FINITE) >= 8          # two 32-bit counters
    assert ws(srnl.FLAG_CHECK_FINITE, B=0) == 0     # empty grid
    assert ws(srnl.FLAG_CHECK_FINITE, C=12) == 0    # invalid shape
    assert L.srnl_scan_workspace_bytes(1, 2, 2, 8, 2, 4, 15, None) == 0
    # the forward record: only where the windowed backward applies (d = 32,
    # readout after the write), 256-byte aligned, counters after it
    rec = ws(srnl.FLAG_RECORD, C=64, heads=2, d=32)
    assert rec > 0 and rec % 256 == 0
    assert ws(srnl.FLAG_RECORD | srnl.FLAG_CHECK_FINITE, C=64, heads=2, d=32) == rec + 256
    assert ws(srnl.FLAG_RECORD | srnl.FLAG_READ_BEFORE, C=64, heads=2, d=32) == 0
    assert ws(srnl.FLAG_RECORD, C=32, heads=2, d=16) == 0
    # with the record given, the backward's own workspace is smaller
    p0 = srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, 0, None)
    p1 = srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, srnl.FLAG_RECORD, None)
    b0 = L.srnl_scan_bwd_workspace_bytes(2, 3, 4, 64, 2, 32, 15, ctypes.byref(p0))
    b1 = L.srnl_scan_bwd_workspace_bytes(2, 3, 4, 64, 2, 32, 15, ctypes.byref(p1))
    assert 0 < b1 < b0 and b0 - b1 <= rec
    # an empty grid is a no-op with the check as without it
    assert _scan(B=0, flags=srnl.FLAG_CHECK_FINITE) == srnl.SRNL_OK


def _scan_1d(x=0, B=1, N=4, C=8, heads=2, d=4, **kw):
    p = srnl.Params(None, None, kw.pop("in_dtype", 0), kw.pop("alpha_max", 0.9),
                    kw.pop("eps", 1e-6), kw.pop("chunk_row", 0), 0, kw.pop("flags", 0), None)
    return srnl.lib().srnl_scan_1d(x, B, N, C, heads, d, ctypes.byref(p), None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=12, C=24), srnl.SRNL_ERR_ARG),          # head dim not allowed
    (dict(C=12), srnl.SRNL_ERR_ARG),                # C != heads * d
    (dict(N=-1), srnl.SRNL_ERR_ARG),
    (dict(B=-1), srnl.SRNL_ERR_ARG),
    (dict(chunk_row=-3), srnl.SRNL_ERR_ARG),
    (dict(alpha_max=1.0), srnl.SRNL_ERR_ARG),
    (dict(in_dtype=7), srnl.SRNL_ERR_DTYPE),
])
def test_scan_1d_argument_errors(kw, status):
    assert _scan_1d(**kw) == status


def test_scan_1d_null_params_and_empty_sequence():
    L = srnl.lib()
    assert L.srnl_scan_1d(None, 1, 4, 8, 2, 4, None, None) == srnl.SRNL_ERR_PTR
    assert _scan_1d(N=0) == srnl.SRNL_OK      # empty sequence: no-op, no pointer needed
    assert _scan_1d(B=0) == srnl.SRNL_OK
    assert L.srnl_scan_1d_bwd(None, 1, 4, 8, 2, 4, None, None, None, 0, None, None,
                              None) == srnl.SRNL_ERR_PTR
    p = srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, 0, None)
    assert L.srnl_scan_1d_bwd(None, 0, 4, 8, 2, 4, ctypes.byref(p), None, None, 0, None, None,
                              None) == srnl.SRNL_OK
    assert L.srnl_scan_1d_workspace_bytes(1, 4, 8, 2, 4, None) == 0
    assert L.srnl_scan_1d_bwd_workspace_bytes(1, 4, 8, 2, 4, None) == 0


@pytest.mark.parametrize("chunk", [0, 100])
def test_scan_1d_workspace_queries_apply_the_1d_chunk(chunk):
    """The 1-D queries size the record and the backward's workspace for the
    chunks srnl_scan_1d runs: 64 tokens when chunk_row is 0 (the 2-D query on
    the 1 x N grid would read 0 as one chunk of N tokens)."""
    L = srnl.lib()
    B, N, C, heads, d = 2, 300, 64, 2, 32
    eff = chunk if chunk > 0 else 64
    for flags in (srnl.FLAG_RECORD, srnl.FLAG_RECORD | srnl.FLAG_CHECK_FINITE, 0):
        p1 = srnl.Params(None, None, 0, 0.9, 1e-6, chunk, 0, flags, None)
        p2 = srnl.Params(None, None, 0, 0.9, 1e-6, eff, 0, flags, None)
        a = L.srnl_scan_1d_workspace_bytes(B, N, C, heads, d, ctypes.byref(p1))
        b = L.srnl_scan_workspace_bytes(B, 1, N, C, heads, d, 1, ctypes.byref(p2))
        assert a == b
        a = L.srnl_scan_1d_bwd_workspace_bytes(B, N, C, heads, d, ctypes.byref(p1))
        b = L.srnl_scan_bwd_workspace_bytes(B, 1, N, C, heads, d, 1, ctypes.byref(p2))
        assert a == b and a > 0
    p0 = srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, srnl.FLAG_RECORD, None)
    whole = L.srnl_scan_workspace_bytes(B, 1, N, C, heads, d, 1, ctypes.byref(p0))
    if chunk == 0:
        assert L.srnl_scan_1d_workspace_bytes(B, N, C, heads, d, ctypes.byref(p0)) != whole


def _block(B=1, H=2, W=2, C=64, heads=2, d=32, mask=15, q=None, F=128, eps=1e-5,
           weights=True, params=True):
    p = srnl.Params(None, q, 0, 0.9, 1e-6, 0, 0, 0, None)
    w = srnl.BlockWeights(*([None] * 12), F, eps)
    return srnl.lib().srnl_block_fwd(None, B, H, W, C, heads, d, mask,
                                     ctypes.byref(p) if params else None,
                                     ctypes.byref(w) if weights else None, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(params=False), srnl.SRNL_ERR_PTR),
    (dict(weights=False), srnl.SRNL_ERR_PTR),
    (dict(q=1), srnl.SRNL_ERR_ARG),                   # the block forms its own queries
    (dict(C=48, heads=3, d=16), srnl.SRNL_ERR_ARG),   # block channels not supported
    (dict(C=1024, heads=16, d=64), srnl.SRNL_ERR_ARG),
    (dict(F=40), srnl.SRNL_ERR_ARG),                  # hidden width not a multiple of 32
    (dict(F=0), srnl.SRNL_ERR_ARG),
    (dict(eps=0.0), srnl.SRNL_ERR_ARG),
    (dict(C=60, heads=2, d=30), srnl.SRNL_ERR_ARG),   # head dim
])
def test_block_argument_errors(kw, status):
    assert _block(**kw) == status
    assert srnl.lib().srnl_last_error().decode() != ""


def test_block_empty_grid_is_a_no_op():
    assert _block(B=0) == srnl.SRNL_OK
    assert srnl.lib().srnl_block_workspace_bytes(0, 2, 2, 64, 15) == 0
    # u, q, s planes and four route planes, each 64-float aligned
    assert srnl.lib().srnl_block_workspace_bytes(1, 2, 3, 64, 15) == 4 * (3 * 384 + 4 * 384)


def test_block_weights_binding_checks_shapes():
    """The library sees only pointers, so the binding checks every block
    parameter's shape and dtype (on CPU tensors: nothing is launched)."""
    import torch
    C, F = 64, 128
    f, b = torch.float32, torch.bfloat16
    bw = dict(ln1_w=torch.ones(C, dtype=f), ln1_b=torch.zeros(C, dtype=f),
              wq=torch.zeros(C, C, dtype=b), dw_w=torch.zeros(C, 3, 3, dtype=f),
              dw_b=torch.zeros(C, dtype=f), ln2_w=torch.ones(C, dtype=f),
              ln2_b=torch.zeros(C, dtype=f), w1=torch.zeros(F, C, dtype=b),
              b1=torch.zeros(F, dtype=f), w2=torch.zeros(C, F, dtype=b), b2=torch.zeros(C, dtype=f))
    sc = torch.ones(4, C, dtype=f)
    w = srnl.block_weights(bw, sc)
    assert w.ffn_hidden == F and w.channels == C
    for k, bad in (("w2", torch.zeros(C, F + 32, dtype=b)), ("w1", torch.zeros(F, C, dtype=f)),
                   ("dw_w", torch.zeros(C, 9, dtype=f)), ("b1", torch.zeros(F + 1, dtype=f))):
        with pytest.raises(ValueError):
            srnl.block_weights(dict(bw, **{k: bad}), sc)
    with pytest.raises(ValueError):
        srnl.block_weights(bw, torch.ones(4, C + 4, dtype=f))


def test_binding_checks_buffer_shapes():
    """The binding rejects mis-shaped states, outputs and gradients before
    calling the library (CPU tensors: the checks come first)."""
    import torch
    x = torch.zeros(1, 4, 4, 64)
    st = torch.zeros(4, 2, 3 * 32 * 32 + 2 * 32)
    with pytest.raises(ValueError):
        srnl.scan_fwd(x, st[:, :1], 2, 32, 15)              # one head's states for two heads
    with pytest.raises(ValueError):
        srnl.scan_fwd(x, st, 2, 32, 15, out=torch.zeros(3, 1, 16, 64))
    with pytest.raises(ValueError):
        srnl.fuse(torch.zeros(4, 1, 16, 64), 1, 4, 4, 64, 15, torch.zeros(4, 32))
    with pytest.raises(ValueError):
        srnl.scan_bwd(x, st, 2, 32, torch.zeros(2, 1, 16, 64), 15)
    with pytest.raises(ValueError):
        srnl.fuse_bwd(torch.zeros(1, 4, 4, 32), torch.zeros(4, 1, 16, 64), 1, 4, 4, 64, 15,
                      torch.zeros(4, 64))
    with pytest.raises(ValueError):
        srnl.scan_1d(torch.zeros(1, 10, 64), st, 2, 32)     # 1-D states are [heads][...]


def test_fuse_bwd_noalloc_rejects_sizes_beyond_its_scratch_before_any_device_work():
    """4 routes x ceil(700 * 56 * 56 / 256) blocks x 64 channels x 4 bytes of
    partial sums exceed the library's 8 MiB scratch: a workspace error,
    returned before the pointers are looked at."""
    L = srnl.lib()
    assert L.srnl_fuse_bwd_noalloc(None, None, 700, 56, 56, 64, 15, None, None, None,
                                   None) == srnl.SRNL_ERR_WORKSPACE
    assert "scratch" in L.srnl_last_error().decode()


def test_scan_fuse_bwd_workspace_and_argument_errors():
    # the one-call backward: its workspace holds the scan backward's and the
    # fusion backward's partial sums, plus the route gradients only where
    # the windowed d = 32 adjoint (which forms them itself) does not run
    L = srnl.lib()

    def p(flags=0):
        return srnl.Params(None, None, 0, 0.9, 1e-6, 0, 0, flags, None)

    def sizes(B, H, W, heads, d, flags=0, mask=15):
        C, R = heads * d, bin(mask).count("1")
        pp = p(flags)
        one = L.srnl_scan_fuse_bwd_workspace_bytes(B, H, W, C, heads, d, mask, ctypes.byref(pp))
        scan = L.srnl_scan_bwd_workspace_bytes(B, H, W, C, heads, d, mask, ctypes.byref(pp))
        fuse = L.srnl_fuse_bwd_workspace_bytes(B, H, W, C, mask)
        return one, scan, fuse, 4 * R * B * H * W * C

    one, scan, fuse, dyr = sizes(2, 9, 11, 2, 32)
    assert scan + fuse <= one < scan + fuse + dyr
    for d, heads, flags in ((16, 2, 0), (32, 2, srnl.FLAG_READ_BEFORE), (64, 1, 0)):
        one, scan, fuse, dyr = sizes(2, 9, 11, heads, d, flags)
        assert one >= scan + fuse + dyr
    one, scan, fuse, dyr = sizes(1, 5, 7, 2, 32, mask=0b0101)
    assert scan + fuse <= one < scan + fuse + dyr
    pp = p()
    assert L.srnl_scan_fuse_bwd_workspace_bytes(0, 4, 4, 64, 2, 32, 15, ctypes.byref(pp)) == 0
    assert L.srnl_scan_fuse_bwd_workspace_bytes(1, 4, 4, 60, 2, 32, 15, ctypes.byref(pp)) == 0
    assert L.srnl_scan_fuse_bwd_workspace_bytes(1, 4, 4, 64, 2, 32, 15, None) == 0
    # invalid arguments are reported before any device work
    args = (None, None, None, None, 0, None, None, None, None)
    assert L.srnl_scan_fuse_bwd(None, 1, 4, 4, 60, 2, 32, 15, ctypes.byref(pp), *args) == srnl.SRNL_ERR_ARG
    assert L.srnl_scan_fuse_bwd(None, 1, 4, 4, 64, 2, 12, 15, ctypes.byref(pp), *args) == srnl.SRNL_ERR_ARG
    assert L.srnl_scan_fuse_bwd(None, 1, 4, 4, 64, 2, 32, 15, None, *args) == srnl.SRNL_ERR_PTR
    assert L.srnl_scan_fuse_bwd(None, 0, 4, 4, 64, 2, 32, 15, ctypes.byref(pp), *args) == srnl.SRNL_OK
    # too small a workspace
    assert L.srnl_scan_fuse_bwd(None, 1, 4, 4, 64, 2, 32, 15, ctypes.byref(pp), None, None, None,
                                None, 16, None, None, None, None) == srnl.SRNL_ERR_WORKSPACE
