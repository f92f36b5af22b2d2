"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m rejection_sampling_verify_sample_amd.build [-v]
       python -m rejection_sampling_verify_sample_amd.build --asan-host OUT.so   (host code under AddressSanitizer)
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


# The host code (argument checks, workspace layout, launches) instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (any finding aborts); the device code
# is built as usual. Load it with the sanitizer's runtime preloaded (asan_runtime())
# and ASAN_OPTIONS=detect_leaks=0 (the Python interpreter's own allocations are not
# this library's).
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-shared-libasan"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime ('' when absent)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or ""
    if not clang:
        return ""
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def build_asan_host(out_path: str, verbose: bool = False) -> str:
    """Compile every HIP source into out_path with the host code under AddressSanitizer."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    flags = HIPCC_FLAGS + ["-Xarch_host", "-g"] + ASAN_HOST_FLAGS
    cmd = [hipcc(), *flags, "-o", out_path, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr}")
    return out_path


if __name__ == "__main__":
    if "--asan-host" in sys.argv:
        print(build_asan_host(sys.argv[sys.argv.index("--asan-host") + 1], verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
