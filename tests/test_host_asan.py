"""The library's host code under AddressSanitizer (CPU only, no GPU).

libsrnl is rebuilt with the sanitizer on its host pass only (the device code
is compiled as usual and never runs here), and tests/host_asan_driver.c
drives every entry point along the paths that return before any device
work: argument validation, empty grids, workspace sizing with overflowing
sizes, NULL pointers, and the host helpers over whole grids. A memory error
in that code makes the sanitizer abort the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_under_address_sanitizer(tmp_path):
    lib = tmp_path / "libsrnl_asan.so"
    drv = tmp_path / "driver"
    src = os.path.join(ROOT, "self_referential_memory_amd", "csrc", "srnl.hip")
    inc = os.path.join(ROOT, "include")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", inc, "-o", str(lib), src],
                   check=True, capture_output=True, timeout=600)
    subprocess.run([CLANG, "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I", inc,
                    os.path.join(ROOT, "tests", "host_asan_driver.c"), "-L", str(tmp_path),
                    "-lsrnl_asan", f"-Wl,-rpath,{tmp_path}", "-o", str(drv)],
                   check=True, capture_output=True, timeout=120)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([str(drv)], capture_output=True, text=True, timeout=120, env=env)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == "ok"
    shutil.rmtree(tmp_path, ignore_errors=True)
