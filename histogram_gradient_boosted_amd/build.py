"""Build the HIP library libhgb.so in-tree for gfx950 (hipcc cross-compiles
without a GPU).  `python -m histogram_gradient_boosted_amd.build` or build()."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhgb.so")
SOURCES = [os.path.join(CSRC, "hgb.hip")]
# the LDS atomic-rate microbenchmark that bench.py reports beside the fill
PROBE_LIB = os.path.join(PKG, "liblds_rate.so")
PROBE_SOURCES = [os.path.join(CSRC, "lds_rate.hip")]
HEADERS = [os.path.join(CSRC, "hgb_kernels.h"), os.path.join(CSRC, "hgb_layout.h"), os.path.join(CSRC, "hgb_plan.h"),
           os.path.join(INCLUDE, "hgb.h")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the split scan's fp64 gain is evaluated exactly as written
    "-ffp-contract=off",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE,
]


def _compile(lib: str, sources, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile libhgb.so and the LDS-rate microbenchmark library."""
    _compile(LIB, SOURCES, verbose)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
