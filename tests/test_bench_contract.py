"""bench.py's command-line contract, CPU only (nothing here touches a GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_counter_passes_fit_the_hardware_limits():
    """Each rocprofv3 --pmc pass stays within one run's counter budget: at
    most 8 SQ, 4 TCC (FETCH_SIZE takes 3, WRITE_SIZE 2), 2 GRBM counters."""
    r = _run("--pmc-passes")
    assert r.returncode == 0
    passes = [l.split() for l in r.stdout.strip().splitlines()]
    assert {p[0] for p in passes} >= {"fetch", "write", "mfma", "insts"}
    for name, *counters in passes:
        sq = sum(c.startswith("SQ_") for c in counters)
        tcc = sum(c.startswith("TCC_") for c in counters)
        tcc += 3 * counters.count("FETCH_SIZE") + 2 * counters.count("WRITE_SIZE")
        grbm = sum(c.startswith("GRBM_") for c in counters)
        assert sq <= 8 and tcc <= 4 and grbm <= 2, (name, counters)


def test_committed_counter_digest_matches_the_kernel_sources():
    """The PMC digest under profiles/ was taken on the committed kernel
    sources, so the benchmark line reports its traffic."""
    sys.path.insert(0, ROOT)
    import bench
    d = json.load(open(bench.COUNTERS_FILE))
    assert d["kernel_source_sha"] == bench.src_sha()
    assert d["scan_kernel"]["hbm_bytes_per_launch"] > 0
