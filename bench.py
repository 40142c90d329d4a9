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
COUNTERS_FILE = os.path.join(PROFILES, "hier56_pmc_counters.json")
SRC = os.path.join(ROOT, "self_referential_memory_amd", "csrc", "srnl.hip")

# Published MI355X peaks used for the rooflines (dense MFMA fp32 and bf16)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
CU_NUM = 256
XCDS = 8                        # GRBM_GUI_ACTIVE reads as the sum over the XCDs
PCT_REPS = 50                   # per-step samples behind the median and p10/p90
COPY_PROBE_BYTES = 1 << 30      # one plain device-to-device copy of 1 GiB ...
COPY_PROBE_REPS = 3             # ... done this many times after the timed steps

# Counter passes over this script (one rocprofv3 --pmc run each, with
# --steps 3 --warmup 1 --no-cpu-baseline --copy-probe), digested by
# --pmc-summary into COUNTERS_FILE.
PMC_PASSES = (
    ("fetch", ("FETCH_SIZE",)),
    ("write", ("WRITE_SIZE",)),
    ("tcc_rd", ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                "TCC_EA0_RDREQ_128B_sum")),
    ("tcc_wr", ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")),
    ("mfma", ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F32",
              "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")),
    ("insts", ("SQ_INSTS_VALU_MFMA_F32", "SQ_INSTS_VALU_MFMA_BF16", "SQ_LDS_BANK_CONFLICT",
               "SQ_LDS_IDX_ACTIVE")),
    ("valu", ("SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
              "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")),
)
KERNEL_KEYS = (("scan_kernel", "scan_mfma_kernel<32"), ("fuse_kernel", "fuse_kernel"),
               ("gather_kernel", "gather_kernel"))


def algorithmic_flops_per_unit(d: int) -> int:
    """Work per token x head x route of the plain five-memory form, with a
    fused multiply-add counted as 2 flops: generation and learning signals
    10 d^2 + 8 d (dense contractions) plus the token-order update and readout
    17 d^2 + 20 d."""
    return (10 * d * d + 8 * d) + (17 * d * d + 20 * d)


def algorithmic_bytes(wl, R: int) -> dict:
    """Bytes each kernel of the step must move at least, bf16 input: the scan
    reads x once per route and writes the fp32 route outputs; the fuse reads
    those and writes the bf16 map; the gather reads x and writes R bf16
    copies in route order."""
    n = wl.B * wl.H * wl.W * wl.C
    st = 4 * wl.heads * (3 * wl.d * wl.d + 2 * wl.d) * 4
    return {"scan_kernel": R * n * 2 + st + R * n * 4,
            "fuse_kernel": R * n * 4 + R * wl.C * 4 + n * 2,
            "gather_kernel": n * 2 + R * n * 2}


def src_sha() -> str:
    """sha256 prefix of the library's kernel sources: every file of csrc/ in
    name order, concatenated."""
    d = os.path.dirname(SRC)
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".inc")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def load_counters():
    """The committed counter digest, if it was taken on the current kernel
    source; else None."""
    try:
        t = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_sha") == src_sha() else None


def pmc_summary(root: str, command: str) -> None:
    """Digest the rocprofv3 runs under root (one directory per PMC_PASSES
    entry holding run_counter_collection.csv, plus ktrace/run_kernel_stats.csv
    from a --kernel-trace --stats run) into COUNTERS_FILE.

    HBM bytes: FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    same counter reads for the copy probe (the sum over all copy dispatches
    against COPY_PROBE_REPS x 1 GiB each way); cross-checked against the raw
    TCC-to-memory request counts by size (32, 64, 128 B reads; 32, 64 B
    writes). MFMA: SQ_INSTS_VALU_MFMA_MOPS_* count MFMA work in units of 512
    flops; utilisation is that work at the published dense peak of its type,
    over the kernel's average duration."""
    import collections
    import csv

    def read(name):
        path = os.path.join(root, name, "run_counter_collection.csv")
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(path)):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return agg

    def per_kernel(agg, key):
        rows = [v for k, v in agg.items() if key in k]
        if not rows:
            return None
        return {c: sum(x) / len(x) for c, x in rows[0].items()}

    def total(agg, key, counter):
        return sum(sum(v[counter]) for k, v in agg.items() if key in k)

    passes = {name: read(name) for name, _ in PMC_PASSES}
    stats = {}
    with open(os.path.join(root, "ktrace", "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            stats[r["Name"]] = r
    dur = {}
    for name, key in KERNEL_KEYS:
        row = next((v for k, v in stats.items() if key in k), None)
        dur[name] = None if row is None else float(row["AverageNs"]) * 1e-9
    probe = COPY_PROBE_BYTES * COPY_PROBE_REPS
    f_scale = probe / (total(passes["fetch"], "copyBuffer", "FETCH_SIZE") * 1024.0)
    w_scale = probe / (total(passes["write"], "copyBuffer", "WRITE_SIZE") * 1024.0)
    out = {"kernel_source_sha": src_sha(), "command": command,
           "copy_probe": {"bytes_each_way": probe, "fetch_scale": f_scale,
                          "write_scale": w_scale}}
    for name, key in KERNEL_KEYS:
        F = per_kernel(passes["fetch"], key)
        if F is None:
            continue
        Wr = per_kernel(passes["write"], key)
        rd = per_kernel(passes["tcc_rd"], key)
        wr = per_kernel(passes["tcc_wr"], key)
        fb = F["FETCH_SIZE"] * 1024.0 * f_scale
        wb = Wr["WRITE_SIZE"] * 1024.0 * w_scale
        k = {"average_duration_s": dur[name],
             "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
             "hbm_bytes_per_launch": fb + wb,
             "raw": {"FETCH_SIZE_KiB": F["FETCH_SIZE"], "WRITE_SIZE_KiB": Wr["WRITE_SIZE"]}}
        if rd is not None and wr is not None:
            n32, n64 = rd["TCC_EA0_RDREQ_32B_sum"], rd["TCC_EA0_RDREQ_64B_sum"]
            n128, nrd = rd["TCC_EA0_RDREQ_128B_sum"], rd["TCC_EA0_RDREQ_sum"]
            w64, nwr = wr["TCC_EA0_WRREQ_64B_sum"], wr["TCC_EA0_WRREQ_sum"]
            k["request_bytes"] = {"read": 32 * n32 + 64 * n64 + 128 * n128,
                                  "write": 64 * w64 + 32 * (nwr - w64)}
            k["raw"].update({"rd_req": nrd, "rd_32B": n32, "rd_64B": n64, "rd_128B": n128,
                             "wr_req": nwr, "wr_64B": w64})
        if dur[name]:
            k["hbm_GBs"] = (fb + wb) / dur[name] / 1e9
        v = per_kernel(passes["valu"], key)
        if v is not None:
            # rocprof's VALUBusy: quad-cycles of VALU work summed over the
            # SIMDs (four per CU), per CU, over the active cycles of one XCD
            cyc = v["GRBM_GUI_ACTIVE"] / XCDS
            k["valu"] = {"busy": v["SQ_ACTIVE_INST_VALU"] / CU_NUM / cyc,
                         "lds_busy": v["SQ_ACTIVE_INST_LDS"] / CU_NUM / cyc,
                         "wait_inst_frac": v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"],
                         "active_inst_frac": v["SQ_ACTIVE_INST_ANY"] / v["SQ_WAVE_CYCLES"],
                         "raw": v}
        m = per_kernel(passes["mfma"], key)
        extra = per_kernel(passes["insts"], key)
        if m is not None and extra is not None:
            m = dict(m, **extra)
        if m is not None and dur[name]:
            f32 = 512.0 * m["SQ_INSTS_VALU_MFMA_MOPS_F32"]
            bf16 = 512.0 * m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
            t = dur[name]
            k["mfma"] = {
                "f32_flops": f32, "bf16_flops": bf16,
                "f32_TFLOPs": f32 / t / 1e12, "bf16_TFLOPs": bf16 / t / 1e12,
                "pipe_util": (f32 / (PEAK_FP32_MFMA_TFLOPS * 1e12)
                              + bf16 / (PEAK_BF16_MFMA_TFLOPS * 1e12)) / t,
                "raw": m}
        out[name] = k
    out["hbm_bytes_per_launch"] = out["scan_kernel"]["hbm_bytes_per_launch"]
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(out, open(COUNTERS_FILE, "w"), indent=2)
    print(json.dumps(out, indent=2))


def host_cpu() -> dict:
    """The host's CPU model (lscpu, else /proc/cpuinfo) and core counts."""
    import subprocess
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": aff}


def oracle_threads() -> int:
    """Threads for the all-core oracle figure: the cores this process may run
    on, at most 16 (a one-GPU machine's CPU share)."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, aff or 1))


def cpu_baseline(wl, n_items: int):
    """The oracle, unchanged, on batch items 0..n_items-1: once on one thread
    (the reported value) and once with the batch split over oracle_threads()
    threads (the all-core figure; ctypes releases the GIL, each thread runs
    the single-threaded oracle on its own items). Returns the record and the
    all-core run's route outputs."""
    import numpy as np
    import oracle
    n_items = min(n_items, wl.B)
    sample = wl.x[:n_items]
    kw = dict(alpha_max=wl.alpha_max, eps=wl.eps)
    t0 = time.perf_counter()
    y = oracle.scan(sample, wl.states, wl.heads, wl.d, 15, **kw)
    oracle.fuse(y, n_items, wl.H, wl.W, wl.C, 15, wl.scales)
    dt = time.perf_counter() - t0
    nt = oracle_threads()
    t1 = time.perf_counter()
    ya = oracle.scan(sample, wl.states, wl.heads, wl.d, 15, threads=nt, **kw)
    oracle.fuse(ya, n_items, wl.H, wl.W, wl.C, 15, wl.scales)
    dta = time.perf_counter() - t1
    assert np.array_equal(y, ya)
    units = n_items * wl.H * wl.W * wl.heads
    what = ("the whole batch" if n_items == wl.B else
            f"batch items 0..{n_items - 1} of {wl.B}")
    rec = {"value": units / dt, "unit": "tokens·heads/s", "cores": 1, "kind": "oracle",
           "sample": f"{what} (all 4 routes, {wl.heads} heads, {wl.H}x{wl.W}), scan + fuse, "
                     f"single-threaded double-precision oracle, {dt:.1f} s",
           "all_cores": {"value": units / dta, "cores": nt, "seconds": dta,
                         "how": "the same oracle on the same items, batch split over "
                                f"{nt} threads"}}
    rec.update(host_cpu())
    return rec, ya


def oracle_check(wl, yg, fused_g, yo) -> dict:
    """Largest error of the GPU's route outputs (yg, [R][n][N][C] for the
    first n batch items) against the oracle's (yo): globally per route slot
    (max |g - o| / max |o|), per chunk on each live chunk's own scale, and of
    the fused output in its stored dtype."""
    import numpy as np
    import oracle
    n = yo.shape[1]
    glob, chunk = 0.0, 0.0
    for s in range(yo.shape[0]):
        o, g = yo[s], yg[s]
        glob = max(glob, float(np.abs(g - o).max() / np.abs(o).max()))
        L = wl.chunk_row or wl.W if s < 2 else wl.chunk_col or wl.H
        for c0 in range(0, wl.N, L):
            m = np.abs(o[:, c0:c0 + L]).max(axis=(1, 2))
            e = np.abs(g[:, c0:c0 + L] - o[:, c0:c0 + L]).max(axis=(1, 2))
            live = m > 1e-20
            if live.any():
                chunk = max(chunk, float((e[live] / m[live]).max()))
    fo = oracle.fuse(yo, n, wl.H, wl.W, wl.C, 15, wl.scales)
    ef = float(np.abs(fused_g[:n] - fo).max() / np.abs(fo).max())
    return {"items": n, "max_rel_err_routes": glob, "max_rel_err_chunk": chunk,
            "max_rel_err_fused_bf16": ef, "bars": {"routes": 1e-4, "fused_bf16": 2e-2}}


def control_activity(wl, n_items: int) -> dict:
    """How often the two stability controls act on the timed workload, from
    the oracle's per-token trace over batch items 0..n_items-1, per token x
    head x route: the injection cap is active where eta g > 1 - alpha (the
    uncapped step would leave the margin; the hard-clamp ablation would cut
    it there), the spectral clamp where it lowers the capped step."""
    import numpy as np
    import oracle
    n = min(n_items, wl.B)
    _, tr = oracle.scan(wl.x[:n], wl.states, wl.heads, wl.d, 15, alpha_max=wl.alpha_max,
                        eps=wl.eps, trace=True, threads=oracle_threads())
    alpha, eta, eta1, eta2, g = (tr[..., k] for k in (10, 11, 12, 13, 14))
    return {"items": n, "units": int(alpha.size),
            "cap_active_frac": float((eta * g > 1.0 - alpha).mean()),
            "clamp_active_frac": float((eta2 < eta1).mean()),
            "soft_cap_mean_ratio": float((eta1 / eta).mean())}


def percentiles(v) -> dict:
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "n": int(a.size)}


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


def main_stages(args):
    """Forward (scan + fuse, four routes) on every stage shape: the four
    hierarchical stages at batch 64 (56x56/C=64/2 heads, 28x28/C=128/4,
    14x14/C=256/8, 7x7/C=512/16, d=32, N(0,1), seed 3), the plain-backbone
    map (batch 32, 14x14, C=192, 3 heads x d=64, seed 1) and the
    dense-prediction map (batch 2, 200x304, C=64, 2 heads x d=32, 5 % of the
    tokens x50, seed 4); bf16 input, fp32 state. value = tokens*heads/s of
    one pass over the four hierarchical stages."""
    import torch
    from self_referential_memory_amd import srnl, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wls = synth.hier_sweep() + [synth.plain14(), synth.dense200x304()]
    stages = []
    for wl in wls:
        x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
        st = torch.from_numpy(wl.states).to(dev)
        sc = torch.from_numpy(wl.scales).to(dev)
        y = torch.empty((4, wl.B, wl.N, wl.C), dtype=torch.float32, device=dev)
        out = torch.empty((wl.B, wl.H, wl.W, wl.C), dtype=torch.bfloat16, device=dev)
        p = srnl.make_params(st, x, alpha_max=wl.alpha_max, eps=wl.eps,
                             chunk_row=wl.chunk_row, chunk_col=wl.chunk_col)
        steps = args.steps
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
               for _ in range(steps)]
        for i in range(args.warmup + steps):
            e = evs[i - args.warmup] if i >= args.warmup else None
            if e is not None:
                e[0].record()
            srnl.scan_fwd(x, st, wl.heads, wl.d, 15, out=y, params=p)
            if e is not None:
                e[1].record()
            srnl.fuse(y, wl.B, wl.H, wl.W, wl.C, 15, sc, out=out)
            if e is not None:
                e[2].record()
        torch.cuda.synchronize()
        scan_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        step_ms = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
        units = wl.B * wl.N * wl.heads
        flops = algorithmic_flops_per_unit(wl.d) * units * 4
        stages.append({"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C,
                       "heads": wl.heads, "d": wl.d, "chains": 4 * wl.B * wl.heads,
                       "chunk": [wl.chunk_row or wl.W, wl.chunk_col or wl.H],
                       "ms_per_step": step_ms, "scan_ms": scan_ms,
                       "tokens_heads_per_s": units / (step_ms / 1000.0),
                       "mfma_frac": flops / (scan_ms / 1000.0) / 1e12 / PEAK_FP32_MFMA_TFLOPS})
        print(f"[stage] {wl.name}: {step_ms:.3f} ms/step, scan {scan_ms:.3f} ms", file=sys.stderr,
              flush=True)
        del x, y, out
    hier = stages[:4]
    tot_units = sum(s["B"] * s["H"] * s["W"] * s["heads"] for s in hier)
    tot_ms = sum(s["ms_per_step"] for s in hier)
    rec = {"metric": "SRNL fwd tokens·heads/s (4 routes), one pass over the hierarchical stages",
           "value": tot_units / (tot_ms / 1000.0), "unit": "tokens·heads/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": tot_ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "stages: hierarchical sweep 56/28/14/7 at batch 64, plus "
                                  "plain14 and dense200x304 (reported per stage)",
                      "parallelism": "single GPU"},
           "stages": stages}
    print(json.dumps(rec), flush=True)


def block_flops_per_token(C: int, F: int) -> int:
    """Algorithmic flops of the block around the operator, per token (FMA =
    2): the query projection 2C^2, the depthwise 3x3 2*9C, the feed-forward
    network 4CF; the norms, GELU and residual adds are left out."""
    return 2 * C * C + 18 * C + 4 * C * F


def main_block56(args):
    """One residual block around the operator (srnl_block_fwd) at the
    hierarchical stage-1 shape: B=64, 56x56, C=64 = 2 heads x d=32, FFN
    hidden 256, bf16 input (AR(1) rows, seed 2), block parameters seed 2.
    value = tokens/s of the whole block. The scan and the fusion are then
    timed again on the block's own u and q (left in its workspace), and the
    block's two kernels are given the remainder."""
    import numpy as np
    import torch
    from self_referential_memory_amd import srnl, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.hier56()
    F = 256
    bw = synth.block_weights(2, wl.C, F)
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    dw = dict(ln1_w=t(bw.ln1_w), ln1_b=t(bw.ln1_b), wq=t(bw.wq, torch.bfloat16), dw_w=t(bw.dw_w),
              dw_b=t(bw.dw_b), ln2_w=t(bw.ln2_w), ln2_b=t(bw.ln2_b), w1=t(bw.w1, torch.bfloat16),
              b1=t(bw.b1), w2=t(bw.w2, torch.bfloat16), b2=t(bw.b2))
    x = t(wl.x, torch.bfloat16)
    st = t(wl.states)
    sc = t(wl.scales)
    w = srnl.block_weights(dw, sc, bw.ln_eps)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    nbytes = srnl.lib().srnl_block_workspace_bytes(B, H, W, C, 15)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    out = torch.empty_like(x)
    p = srnl.make_params(st, x)

    def step():
        srnl.block_fwd(x, st, w, wl.heads, wl.d, 15, out=out, workspace=ws, params=p)

    def timed(fn, steps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = timed(step, args.steps)
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    # the operator and the fusion alone, on the block's u and q
    plane = (B * H * W * C + 63) // 64 * 64
    u = ws[:B * H * W * C].view(B, H, W, C)
    q = ws[plane:plane + B * H * W * C].view(B, H, W, C)
    y = ws[3 * plane:3 * plane + 4 * B * H * W * C].view(4, B, H * W, C)
    sf = torch.empty((B, H, W, C), dtype=torch.float32, device=dev)
    pq = srnl.make_params(st, u, q)
    scan_ms = timed(lambda: srnl.scan_fwd(u, st, wl.heads, wl.d, 15, out=y, params=pq), args.steps)
    fuse_ms = timed(lambda: srnl.fuse(y, B, H, W, C, 15, sc, out=sf), args.steps)
    ntok = B * H * W
    units = ntok * wl.heads
    srnl_flops = algorithmic_flops_per_unit(wl.d) * units * 4
    blk_flops = block_flops_per_token(C, F) * ntok
    achieved = srnl_flops / (scan_ms / 1000.0) / 1e12
    rest_ms = step_ms - scan_ms - fuse_ms
    # the block kernels' compulsory bytes: pre reads x, writes u and q; post
    # reads x, u, s and writes out
    blk_bytes = ntok * C * (2 + 8 + 2 + 4 + 4 + 2)
    rec = {
        "metric": "VisionHOPE block fwd tokens/s (SRNL 4 routes + depthwise branch + FFN)",
        "value": ntok / (ms / 1000.0), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "block56: one residual block at the hierarchical stage-1 shape, "
                               "B=64, 56x56, C=64 = 2 heads x d=32, FFN hidden 256, bf16 input, "
                               "bf16 projection weights, fp32 arithmetic, seed 2",
                   "B": B, "H": H, "W": W, "C": C, "heads": wl.heads, "d": wl.d, "ffn_hidden": F,
                   "routes": 4, "input_dtype": "bf16", "parallelism": "single GPU"},
        "roofline": {"kernel": "scan_kernel (on u with queries q, fp32)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_MFMA_TFLOPS, "traffic": None,
                     "scan_ms": scan_ms, "algorithmic_flops_per_launch": srnl_flops},
        "kernels": {
            "block_step_ms": step_ms, "scan_ms": scan_ms, "fuse_ms": fuse_ms,
            "block_pre_post_ms": rest_ms,
            "block_pre_post_algorithmic_bytes": blk_bytes,
            "block_pre_post_GBs": blk_bytes / (rest_ms / 1000.0) / 1e9 if rest_ms > 0 else None,
            "block_pre_post_algorithmic_flops": blk_flops,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import block as OB
        n = min(args.cpu_items, 8)
        t0 = time.perf_counter()
        OB.block_forward(wl.x[:n], wl.states, wl.scales, bw, wl.heads, wl.d)
        dtc = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": n * H * W / dtc, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"batch items 0..{n - 1} of {B}, the block oracle (the single-threaded "
                      f"double-precision operator oracle plus numpy float64), {dtc:.1f} s"}
    print(json.dumps(rec), flush=True)


def main_bwd(args, wl_name):
    """Backward of a forward step: srnl_scan_fuse_bwd (the results of
    srnl_fuse_bwd + srnl_scan_bwd in one call) for a given dL/d(fused output),
    forward outputs and inputs resident in HBM. hier56:
    the hierarchical stage-1 map (d = 32: recording forward + windowed
    adjoint); plain14: the plain backbone's map (B=32, 14x14, C=192, 3 heads
    of d=64, chunks of 14 tokens: recording forward + the single-window
    adjoint at d = 64)."""
    import numpy as np
    import torch
    from self_referential_memory_amd import srnl, synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.hier56() if wl_name == "hier56" else synth.plain14()
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
    nb_s = L.srnl_scan_fuse_bwd_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                                ctypes.byref(p))
    ws_s = torch.empty(nb_s, dtype=torch.uint8, device=dev)
    dsc = torch.empty((4, wl.C), dtype=torch.float32, device=dev)
    dx = torch.empty((wl.B, wl.H, wl.W, wl.C), dtype=torch.float32, device=dev)
    dst = torch.empty_like(st)
    stream = torch.cuda.current_stream().cuda_stream

    def step(a=None, b=None):
        if a is not None:
            a.record()
        rc = L.srnl_scan_fuse_bwd(x.data_ptr(), wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                  ctypes.byref(p), y.data_ptr(), sc.data_ptr(), dout.data_ptr(),
                                  ws_s.data_ptr(), nb_s, dx.data_ptr(), None, dst.data_ptr(),
                                  dsc.data_ptr())
        if b is not None:
            b.record()
        if rc != 0:
            raise RuntimeError(f"srnl_scan_fuse_bwd failed: {rc}")

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

    # One training step of the operator (forward scan + fuse, fusion backward,
    # scan backward), once with the forward keeping its record for the
    # backward (SRNL_FLAG_RECORD) and once with the backward recording it again.
    pr = srnl.make_params(st, x, flags=srnl.FLAG_RECORD)
    nb_r = L.srnl_scan_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                       ctypes.byref(pr))
    ws_r = torch.empty(nb_r, dtype=torch.uint8, device=dev)
    pr.workspace, pr.workspace_bytes = ws_r.data_ptr(), nb_r
    nb_sr = L.srnl_scan_fuse_bwd_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                                 ctypes.byref(pr))
    ws_sr = torch.empty(nb_sr, dtype=torch.uint8, device=dev)
    fused = torch.empty((wl.B, wl.H, wl.W, wl.C), dtype=torch.bfloat16, device=dev)

    def train(record):
        pp, ws, nb = (pr, ws_sr, nb_sr) if record else (p, ws_s, nb_s)
        rc = L.srnl_scan_fwd(x.data_ptr(), wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                             ctypes.byref(pp), y.data_ptr())
        rc |= L.srnl_fuse(y.data_ptr(), wl.B, wl.H, wl.W, wl.C, 15, sc.data_ptr(),
                          srnl.SRNL_BF16, fused.data_ptr(), stream)
        rc |= L.srnl_scan_fuse_bwd(x.data_ptr(), wl.B, wl.H, wl.W, wl.C, wl.heads, wl.d, 15,
                                   ctypes.byref(pp), y.data_ptr(), sc.data_ptr(), dout.data_ptr(),
                                   ws.data_ptr(), nb, dx.data_ptr(), None, dst.data_ptr(),
                                   dsc.data_ptr())
        if rc != 0:
            raise RuntimeError("training step failed")

    train_ms = {True: None, False: None}
    for record in (() if args.no_train_step else (True, False)):
        for _ in range(args.warmup):
            train(record)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            train(record)
        torch.cuda.synchronize()
        train_ms[record] = (time.perf_counter() - t1) * 1000.0 / args.steps
    units = wl.B * wl.H * wl.W * wl.heads
    flops = 2 * algorithmic_flops_per_unit(wl.d) * units * R
    achieved = flops / (scan_ms / 1000.0) / 1e12
    if wl_name == "hier56":
        what = ("hier56_bwd: backward of the hier56 step (srnl_scan_fuse_bwd), "
                "B=64, 56x56, C=64, 2 heads x d=32, 4 routes")
        kern = ("scan_fuse_bwd (fusion backward partial sums + recording forward + "
                "scan_bwd_wy_kernel reading dout)")
    else:
        what = ("plain14_bwd: backward of the plain14 step (srnl_scan_fuse_bwd), "
                "B=32, 14x14, C=192, 3 heads x d=64, 4 routes")
        kern = ("scan_fuse_bwd (fusion backward + recording forward + "
                "scan_bwd_wy64_kernel)")
    # both scan backwards (recording forward + windowed adjoint) run their
    # contractions on fp32 MFMA
    roof = {"kernel": kern, "bound": "mfma", "achieved": achieved,
            "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA_TFLOPS}
    roof.update({"traffic": None, "call_ms": scan_ms,
                 "timed": "one srnl_scan_fuse_bwd call by HIP events (fusion backward, "
                          "recording forward, adjoint, reductions)",
                 "algorithmic_flops_per_launch": flops})
    rec = {
        "metric": "SRNL bwd tokens·heads/s (4 routes) at stage shapes",
        "value": units / (ms / 1000.0), "unit": "tokens·heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": what,
                   "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads, "d": wl.d,
                   "routes": R, "input_dtype": "bf16", "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": None,
        "train_step": {"what": "srnl_scan_fwd + srnl_fuse (bf16 out) + srnl_scan_fuse_bwd "
                               "per step",
                       "ms_forward_keeps_record": train_ms[True],
                       "ms_backward_records_again": train_ms[False],
                       "record_bytes": nb_r},
    }
    print(json.dumps(rec), flush=True)


PHASES = ("load", "generation", "epilogue", "window_tables", "update", "readout", "refresh")
BWD_PHASES = ("chunk_start_loads", "commit", "dz_and_tables", "unused", "unused",
              "unused", "gin_recurrence", "token_products", "token_dots_tables",
              "token_dq_dk", "scalar_chain", "generation_backward", "chunk_start_refresh")
PHASE_SLOTS = 15


def main_phase_clocks(args):
    """Cycles per phase of the scan kernel, from the phase-clock build of the
    library (python -m self_referential_memory_amd.build --phase-clocks):
    wave 0 of each chain's block stamps the shader clock after every phase's
    closing barrier. One line per workload: mean cycles per sub-block of each
    phase over all chains, and per chain in all."""
    import ctypes
    import numpy as np
    import torch
    from self_referential_memory_amd import build as B_
    from self_referential_memory_amd import srnl, synth
    if not os.path.exists(B_.PHASE_LIB):
        raise RuntimeError(f"{B_.PHASE_LIB} is missing: build it with "
                           "python -m self_referential_memory_amd.build --phase-clocks")
    srnl.LIB_PATH = B_.PHASE_LIB
    L = srnl.lib()
    L.srnl_phase_clocks.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.srnl_phase_clocks.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def read_clocks(nch):
        nb = (nch + 7) // 8 * 8
        buf = np.zeros(nb * PHASE_SLOTS, dtype=np.uint64)
        assert L.srnl_phase_clocks(buf.ctypes.data, buf.size) == 0
        return buf.reshape(nb, PHASE_SLOTS)[:nch].astype(np.float64)

    sweep = synth.hier_sweep()
    wls = [synth.hier56(), synth.hier56(B=32), synth.dense200x304(), sweep[1], sweep[2],
           sweep[3], synth.plain14()]
    for wl in wls:
        x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
        st = torch.from_numpy(wl.states).to(dev)
        y = torch.empty((4, wl.B, wl.N, wl.C), dtype=torch.float32, device=dev)
        for _ in range(3):
            srnl.scan_fwd(x, st, wl.heads, wl.d, 15, out=y)
        torch.cuda.synchronize()
        a = read_clocks(4 * wl.B * wl.heads)
        nsub = float(a[:, PHASE_SLOTS - 2].mean())
        rec = {"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C,
               "heads": wl.heads, "d": wl.d, "chains": a.shape[0], "sub_blocks_per_chain": nsub,
               "cycles_per_chain": float(a[:, PHASE_SLOTS - 1].mean()),
               "cycles_per_sub_block": {k: float(v) for k, v in
                                        zip(PHASES, a[:, :len(PHASES)].mean(axis=0) / nsub)}}
        print(json.dumps(rec), flush=True)
        del x, y
    # the windowed backward of hier56 (its clocks overwrite those of the
    # recording forward that srnl_scan_bwd launches first)
    wl = synth.hier56()
    x = torch.from_numpy(wl.x).to(dev).to(torch.bfloat16)
    st = torch.from_numpy(wl.states).to(dev)
    y = srnl.scan_fwd(x, st, wl.heads, wl.d, 15)
    dy = torch.from_numpy(np.random.default_rng(0).standard_normal(
        tuple(y.shape)).astype(np.float32)).to(dev)
    for _ in range(3):
        srnl.scan_bwd(x, st, wl.heads, wl.d, dy, 15)
    torch.cuda.synchronize()
    a = read_clocks(4 * wl.B * wl.heads)
    nwin = float(a[:, PHASE_SLOTS - 2].mean())
    rec = {"workload": wl.name + "_bwd", "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C,
           "heads": wl.heads, "d": wl.d, "chains": a.shape[0], "windows_per_chain": nwin,
           "cycles_per_chain": float(a[:, PHASE_SLOTS - 1].mean()),
           "cycles_per_window": {k: float(v) for k, v in
                                 zip(BWD_PHASES, a[:, :len(BWD_PHASES)].mean(axis=0) / nwin)}}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-items", type=int, default=64,
                    help="batch items the CPU-baseline oracle runs on (64 = the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle: no CPU baseline, no oracle check, no control activity")
    ap.add_argument("--no-extras", action="store_true",
                    help="hier56: skip the live-state timing and the control-activity trace "
                         "(profiler runs)")
    ap.add_argument("--no-train-step", action="store_true",
                    help="hier56_bwd: skip the training-step timing (kernel traces of the "
                         "backward alone)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (PMC calibration)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="digest the rocprofv3 runs under DIR (one directory per counter "
                         "pass, plus ktrace/) into the committed counter summary")
    ap.add_argument("--pmc-passes", action="store_true",
                    help="print the counter passes, one line each: NAME COUNTER...")
    ap.add_argument("--pmc-command", default="", help="command recorded in the summary")
    ap.add_argument("--phase-clocks", action="store_true",
                    help="cycles per phase of the scan kernel on every stage shape, from the "
                         "phase-clock build of the library")
    ap.add_argument("--workload", choices=("hier56", "seq1d", "hier56_bwd", "plain14_bwd", "stages",
                                           "block56"),
                    default="hier56",
                    help="hier56: the 2-D four-route operator (default); seq1d: the "
                         "standalone 1-D SRNL; hier56_bwd, plain14_bwd: the backward pass on the "
                         "hierarchical stage-1 and the plain-backbone maps; stages: the "
                         "forward on every stage shape; block56: one residual block around "
                         "the operator at the 56x56 shape")
    args = ap.parse_args()
    if args.pmc_passes:
        for name, counters in PMC_PASSES:
            print(name, " ".join(counters))
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.pmc_command)
        return
    if args.phase_clocks:
        main_phase_clocks(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator's chains are independent and would shard over batch, "
              "heads and routes without communication)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "seq1d":
        main_seq1d(args)
        return
    if args.workload == "block56":
        main_block56(args)
        return
    if args.workload in ("hier56_bwd", "plain14_bwd"):
        main_bwd(args, args.workload[:-4])
        return
    if args.workload == "stages":
        main_stages(args)
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

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        srnl.scan_fwd(x, st, wl.heads, wl.d, 15, out=y, params=p)
        if ev is not None:
            ev[1].record()
        srnl.fuse(y, wl.B, wl.H, wl.W, wl.C, 15, sc, out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    scan_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    fuse_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    fused_g = out.double().cpu().numpy() if not args.no_cpu_baseline else None
    y_last = y.double().cpu().numpy() if not args.no_cpu_baseline else None

    # per-step HIP-event samples for the median and p10/p90: the timed steps,
    # then more steps after the timed region until there are PCT_REPS
    more = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
            for _ in range(max(0, PCT_REPS - args.steps))]
    for ev in more:
        step(ev)
    torch.cuda.synchronize()
    samples = list(evs) + more
    timing = {"step_ms": percentiles([e[0].elapsed_time(e[2]) for e in samples]),
              "scan_ms": percentiles([e[0].elapsed_time(e[1]) for e in samples]),
              "fuse_ms": percentiles([e[1].elapsed_time(e[2]) for e in samples]),
              "what": "HIP events on the launch stream around each step (scan + fuse), "
                      f"the {args.steps} timed steps and {len(more)} more after them"}

    # the same launch on states that keep every chunk alive (retention fixed
    # at 0.999, states of std 1): the scan's time does not depend on values
    live = None
    if not args.no_extras:
        wlv = synth.hier56_live()
        xv = torch.from_numpy(wlv.x).to(dev).to(torch.bfloat16)
        stv = torch.from_numpy(wlv.states).to(dev)
        pv = srnl.make_params(stv, xv, alpha_max=wlv.alpha_max, eps=wlv.eps,
                              flags=srnl.FLAG_FIXED_ALPHA)
        for _ in range(3):
            srnl.scan_fwd(xv, stv, wlv.heads, wlv.d, 15, out=y, params=pv)
        lev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
               for _ in range(PCT_REPS)]
        for a, b in lev:
            a.record()
            srnl.scan_fwd(xv, stv, wlv.heads, wlv.d, 15, out=y, params=pv)
            b.record()
        torch.cuda.synchronize()
        lt = percentiles([a.elapsed_time(b) for a, b in lev])
        live = {"workload": "hier56 launch on live states: states of std 1, retention fixed "
                            "at 0.999 (every chunk's output stays O(1))",
                "scan_ms": lt,
                "ratio_to_headline_median": lt["median"] / timing["scan_ms"]["median"]}
        del xv, stv

    # the standalone route gather (not part of the step: the scan gathers its
    # own tokens), timed after the steps for its bandwidth
    g = torch.empty((R, wl.B, wl.N, wl.C), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        srnl.route_gather(x, 15, out=g)
    gev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(10)]
    for a, b in gev:
        a.record()
        srnl.route_gather(x, 15, out=g)
        b.record()
    torch.cuda.synchronize()
    gather_ms = sum(a.elapsed_time(b) for a, b in gev) / len(gev)
    del g

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_PROBE_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()

    ms = dt * 1000.0 / args.steps
    units = wl.B * wl.H * wl.W * wl.heads            # tokens x heads per step
    value = units / (ms / 1000.0)
    thr_units = units * R                            # tokens x heads x routes per launch
    flops = algorithmic_flops_per_unit(wl.d) * thr_units
    achieved = flops / (scan_ms / 1000.0) / 1e12
    prof = load_counters()
    abytes = algorithmic_bytes(wl, R)
    kernels = {}
    for name, k_ms in (("scan_kernel", scan_ms), ("fuse_kernel", fuse_ms),
                       ("gather_kernel", gather_ms)):
        gbs = abytes[name] / (k_ms / 1000.0) / 1e9
        e = {"us": k_ms * 1000.0, "algorithmic_bytes": abytes[name], "achieved_GBs": gbs,
             "peak_GBs": PEAK_HBM_GBS, "hbm_frac": gbs / PEAK_HBM_GBS,
             "pmc_hbm_bytes": None}
        e["valu_busy"] = None
        if prof is not None and name in prof:
            e["pmc_hbm_bytes"] = prof[name]["hbm_bytes_per_launch"]
            if "mfma" in prof[name]:
                e["mfma_pipe_util"] = prof[name]["mfma"]["pipe_util"]
                e["mfma_bf16_TFLOPs_generation_and_grams"] = prof[name]["mfma"]["bf16_TFLOPs"]
            if "valu" in prof[name]:
                e["valu_busy"] = prof[name]["valu"]["busy"]
                e["wait_inst_frac"] = prof[name]["valu"]["wait_inst_frac"]
        kernels[name] = e
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
            "traffic": None if prof is None else prof["hbm_bytes_per_launch"],
            "scan_ms": scan_ms,
            "algorithmic_flops_per_launch": flops,
        },
        "kernels": kernels,
        "timing": timing,
        "value_independence": live,
        "cpu_baseline": None,
        "oracle_check": None,
        "controls": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], yo = cpu_baseline(wl, args.cpu_items)
        rec["oracle_check"] = oracle_check(wl, y_last[:, :yo.shape[1]], fused_g, yo)
        del yo
        if not args.no_extras:
            rec["controls"] = control_activity(wl, args.cpu_items)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
