"""Build libsrnl.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "srnl.hip")
LIB = os.path.join(PKG, "libsrnl.so")
# the same source with the scan kernel's phase clocks compiled in (a
# measurement build, loaded only by bench.py --phase-clocks)
PHASE_LIB = os.path.join(PKG, "libsrnl_phase.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # no packed fp32 instructions (hipcc warns on the host pass: harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs, so that the VALU work between
    # dependent products needs no accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, phase_clocks: bool = False) -> str:
    lib = PHASE_LIB if phase_clocks else LIB
    tmp = lib + ".tmp"
    extra = ["-DSRNL_PHASE_CLOCKS=1"] if phase_clocks else []
    cmd = [HIPCC] + FLAGS + extra + ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_clocks="--phase-clocks" in sys.argv))
