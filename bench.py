#!/usr/bin/env python3
"""Benchmark of the four-route SRNL forward pass on one MI355X.

One step = srnl_scan_fwd (route gather, boundary generation, transition
scalars, token-order update, readout: all four routes) + srnl_fuse (restore and
channel-scale fusion) over one batch of the hierarchical stage-1 grid:
B=64, 56x56, C=64, 2 heads of d=32, chunk 56, bf16 input, fp32 state, rows
AR(1)-correlated (rho = 0.9), seed 2. Inputs are synthetic (synth.hier56) and
resident in HBM before the timed region.

Prints one JSON line with the throughput in tokens*heads/s, the roofline of
the dominant kernel (the scan kernel), and a CPU baseline: the oracle timed on
a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SRNL fwd tokens·heads/s (4 routes) at stage shapes; % of HBM/MFMA roofline"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "scan_kernel_hier56_traffic.json")
SRC = os.path.join(ROOT, "self_referential_memory_amd", "csrc", "srnl.hip")

# Published MI355X peaks used for the roofline (dense fp32 MFMA; the fp32
# vector peak is the same figure).
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def algorithmic_flops_per_unit(d: int) -> int:
    """Work per token x head x route of the plain five-memory form, with a
    fused multiply-add counted as 2 flops: generation and learning signals
    10 d^2 + 8 d (dense contractions) plus the token-order update and readout
    17 d^2 + 20 d."""
    return (10 * d * d + 8 * d) + (17 * d * d + 20 * d)


def src_sha() -> str:
    return hashlib.sha256(open(SRC, "rb").read()).hexdigest()[:16]


def traffic_from_profile(launches_units: int):
    """HBM bytes per scan launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != src_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def pmc_summary(fetch_csv: str, write_csv: str, command: str) -> None:
    """Digest two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, of this
    script with --copy-probe) into profiles/scan_kernel_hier56_traffic.json:
    per-dispatch counter averages, calibrated against the plain 1 GiB device
    copy the probe runs (1 GiB read and 1 GiB written per dispatch)."""
    import csv
    import collections

    def read(path, counter):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    pick = lambda d, key: next(v for k, v in d.items() if key in k)
    gib = float(1 << 30)
    f_scale = gib / (pick(fetch, "copyBuffer") * 1024.0)
    w_scale = gib / (pick(write, "copyBuffer") * 1024.0)
    out = {"kernel_source_sha": src_sha(), "command": command,
           "copy_probe": {"bytes_each_way": int(gib), "fetch_scale": f_scale,
                          "write_scale": w_scale}}
    for key, name in (("scan_mfma_kernel<32", "scan_kernel"), ("fuse_kernel", "fuse_kernel")):
        fb = pick(fetch, key) * 1024.0 * f_scale
        wb = pick(write, key) * 1024.0 * w_scale
        out[name] = {"fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                     "hbm_bytes_per_launch": fb + wb}
    out["hbm_bytes_per_launch"] = out["scan_kernel"]["hbm_bytes_per_launch"]
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=2)
    print(json.dumps(out, indent=2))


def cpu_baseline(wl, n_items: int):
    import numpy as np
    import oracle
    n_items = min(n_items, wl.B)
    sample = wl.x[:n_items]
    t0 = time.perf_counter()
    y = oracle.scan(sample, wl.states, wl.heads, wl.d, 15, alpha_max=wl.alpha_max, eps=wl.eps)
    oracle.fuse(y, n_items, wl.H, wl.W, wl.C, 15, wl.scales)
    dt = time.perf_counter() - t0
    units = n_items * wl.H * wl.W * wl.heads
    what = ("the whole batch" if n_items == wl.B else
            f"batch items 0..{n_items - 1} of {wl.B}")
    return {"value": units / dt, "unit": "tokens·heads/s", "cores": 1, "kind": "oracle",
            "sample": f"{what} (all 4 routes, {wl.heads} heads, {wl.H}x{wl.W}), scan + fuse, "
                      f"single-threaded double-precision oracle, {dt:.1f} s"}


def seq1d_workload():
    """Standalone 1-D SRNL workload: B=256 sequences of 3136 tokens (the
    56x56 token count), C=64 as 2 heads x d=32, bf16 N(0,1) input, default
    64-token chunks, states N(0, 0.02^2), seed 6: 512 independent chains, the
    same chain count as hier56."""
    import numpy as np
    from self_referential_memory_amd import synth
    B, N, C, heads, d = 256, 3136, 64, 2, 32
    x = synth.round_bf16(synth.normals(6, 1, B * N * C).reshape(B, N, C).astype(np.float32))[0]
    st = synth.states(6, heads, d, 0.02)[0]
    return x, st, heads, d


def main_seq1d(args):
    import numpy as np
    import torch
    from self_referential_memory_amd import srnl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xh, sth, heads, d = seq1d_workload()
    B, N, C = xh.shape
    x = torch.from_numpy(xh).to(dev).to(torch.bfloat16)
    st = torch.from_numpy(sth).to(dev)
    y = torch.empty((B, N, C), dtype=torch.float32, device=dev)
    p = srnl.make_params(st, x)
    for _ in range(args.warmup):
        srnl.scan_1d(x, st, heads, d, out=y, params=p)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        srnl.scan_1d(x, st, heads, d, out=y, params=p)
        b.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms = dt * 1000.0 / args.steps
    units = B * N * heads
    flops = algorithmic_flops_per_unit(d) * units
    achieved = flops / (scan_ms / 1000.0) / 1e12
    rec = {
        "metric": "SRNL 1-D fwd tokens·heads/s",
        "value": units / (ms / 1000.0),
        "unit": "tokens·heads/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "seq1d: standalone 1-D SRNL, B=256 sequences x 3136 tokens, "
                               "C=64 = 2 heads x d=32, 64-token chunks, bf16 input, fp32 state, "
                               "seed 6", "B": B, "N": N, "C": C, "heads": heads, "d": d,
                   "chunk": 64, "input_dtype": "bf16", "parallelism": "single GPU"},
        "roofline": {"kernel": "scan_kernel", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_MFMA_TFLOPS, "traffic": None,
                     "scan_ms": scan_ms, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_items, B)
        t0 = time.perf_counter()
        oracle.scan_1d(xh[:n], sth, heads, d)
        dtc = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": n * N * heads / dtc, "unit": "tokens·heads/s", "cores": 1, "kind": "oracle",
            "sample": f"sequences 0..{n - 1} of {B}, single-threaded double-precision oracle, "
                      f"{dtc:.1f} s"}
    print(json.dumps(rec), flush=True)


def main_hier56_bwd(args):
    """Backward of the hier56 step: srnl_fuse_bwd + srnl_scan_bwd for a given
    dL/d(fused output), forward outputs and inputs resident in HBM."""
    import numpy as np
    import torch
    from self_referential_memory_amd import srnl, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.hier56()
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(dev)
    sc = torch.from_numpy(wl.scales).to(dev)
    R = 4
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, 15)
    dout = torch.from_numpy(np.random.default_rng(0).standard_normal(
        (wl.B, wl.H, wl.W, wl.C)).astype(np.float32)).to(dev)
    p = srnl.make_params(st, x)
    L = srnl.lib()
    import ctypes
    nb_s = L.srnl_scan_bwd_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                           ctypes.byref(p))
    nb_f = L.srnl_fuse_bwd_workspace_bytes(wl.B, wl.H, wl.W, wl.C, 15)
    ws_s = torch.empty(nb_s, dtype=torch.uint8, device=dev)
    ws_f = torch.empty(nb_f, dtype=torch.uint8, device=dev)
    dyr = torch.empty_like(y)
    dsc = torch.empty((4, wl.C), dtype=torch.float32, device=dev)
    dx = torch.empty((wl.B, wl.H, wl.W, wl.C), dtype=torch.float32, device=dev)
    dst = torch.empty_like(st)
    stream = torch.cuda.current_stream().cuda_stream

    def step(a=None, b=None):
        L.srnl_fuse_bwd(dout.data_ptr(), y.data_ptr(), wl.B, wl.H, wl.W, wl.C, 15,
                        sc.data_ptr(), dyr.data_ptr(), dsc.data_ptr(), ws_f.data_ptr(), nb_f, stream)
        if a is not None:
            a.record()
        rc = L.srnl_scan_bwd(x.data_ptr(), wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                             ctypes.byref(p), dyr.data_ptr(), ws_s.data_ptr(), nb_s,
                             dx.data_ptr(), None, dst.data_ptr())
        if b is not None:
            b.record()
        if rc != 0:
            raise RuntimeError(f"srnl_scan_bwd failed: {rc}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        step(a, b)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ms = dt * 1000.0 / args.steps
    units = wl.B * wl.H * wl.W * wl.heads
    flops = 2 * algorithmic_flops_per_unit(wl.d) * units * R
    achieved = flops / (scan_ms / 1000.0) / 1e12
    rec = {
        "metric": "SRNL bwd tokens·heads/s (4 routes) at stage shapes",
        "value": units / (ms / 1000.0), "unit": "tokens·heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "hier56_bwd: backward of the hier56 step (srnl_fuse_bwd + "
                               "srnl_scan_bwd), B=64, 56x56, C=64, 2 heads x d=32, 4 routes",
                   "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads, "d": wl.d,
                   "routes": R, "input_dtype": "bf16", "parallelism": "single GPU"},
        "roofline": {"kernel": "scan_bwd_kernel", "bound": "alu", "achieved": achieved,
                     "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_VALU_TFLOPS, "traffic": None,
                     "scan_ms": scan_ms, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-items", type=int, default=64,
                    help="batch items the CPU-baseline oracle runs on (64 = the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (PMC calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="digest two rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--pmc-command", default="", help="command recorded in the summary")
    ap.add_argument("--workload", choices=("hier56", "seq1d", "hier56_bwd"), default="hier56",
                    help="hier56: the 2-D four-route operator (default); seq1d: the "
                         "standalone 1-D SRNL; hier56_bwd: its backward pass")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator's chains are independent and would shard over batch, "
              "heads and routes without communication)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "seq1d":
        main_seq1d(args)
        return
    if args.workload == "hier56_bwd":
        main_hier56_bwd(args)
        return

    import numpy as np
    import torch
    from self_referential_memory_amd import srnl, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.hier56()
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(dev)
    sc = torch.from_numpy(wl.scales).to(dev)
    R = 4
    y = torch.empty((R, wl.B, wl.N, wl.C), dtype=torch.float32, device=dev)
    out = torch.empty((wl.B, wl.H, wl.W, wl.C), dtype=torch.bfloat16, device=dev)
    p = srnl.make_params(st, x, alpha_max=wl.alpha_max, eps=wl.eps)

    def step(ev_a=None, ev_b=None):
        if ev_a is not None:
            ev_a.record()
        srnl.scan_fwd(x, st, wl.heads, wl.d, 15, out=y, params=p)
        if ev_b is not None:
            ev_b.record()
        srnl.fuse(y, wl.B, wl.H, wl.W, wl.C, 15, sc, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        step(a, b)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ms = dt * 1000.0 / args.steps
    units = wl.B * wl.H * wl.W * wl.heads            # tokens x heads per step
    value = units / (ms / 1000.0)
    thr_units = units * R                            # tokens x heads x routes per launch
    flops = algorithmic_flops_per_unit(wl.d) * thr_units
    achieved = flops / (scan_ms / 1000.0) / 1e12
    traffic = traffic_from_profile(thr_units)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "hier56: SRNL forward over the hierarchical stage-1 grid, B=64, "
                        "56x56, C=64, 2 heads x d=32, 4 routes, chunk 56 (rows) / 56 "
                        "(columns), bf16 input, fp32 state and arithmetic, AR(1) rows "
                        "rho=0.9, seed 2",
            "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads, "d": wl.d,
            "routes": R, "input_dtype": "bf16", "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "scan_kernel",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
            "traffic": traffic,
            "scan_ms": scan_ms,
            "algorithmic_flops_per_launch": flops,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_items)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
