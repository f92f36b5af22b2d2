"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m rejection_sampling_verify_sample_amd.build [--check]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "sample.hip", "filter.hip", "greedy.hip", "ngram.hip", "ngram_cache.hip", "ngram_sample.hip",
           "philox.hip", "stats.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # every fused multiply-add is written out; no other contraction changes the rounding
    "-ffp-contract=off",
    # no packed fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libspecverify.so")
    return path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles). Returns the library path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix=".libspecverify.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr}")
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
