"""The library's host code under AddressSanitizer and UBSan (CPU only, no GPU).

The C ABI's argument checks, workspace-size arithmetic and table geometry run on the
host before any HIP call. The library is built once more with that host code
instrumented (the device code as usual), and the ABI tests (tests/test_abi.py) run
against it in a child process with the sanitizer's runtime preloaded; an invalid
host memory access or undefined behaviour (a signed overflow in a size, a shift past
the width) would abort the run with a report.
"""
import os
import subprocess
import sys

import pytest

from rejection_sampling_verify_sample_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

RUNNER = """
import sys
sys.path.insert(0, {root!r})
import rejection_sampling_verify_sample_amd as rsv
import rejection_sampling_verify_sample_amd._lib as L
L.LIB_PATH = rsv.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_checks_are_clean_under_sanitizers(tmp_path):
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:  # no hipcc
        pytest.skip(str(e))
    if not runtime:
        pytest.skip("no AddressSanitizer runtime next to the compiler")
    lib = build.build_asan_host(str(tmp_path / "libspecverify_asan.so"))
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = RUNNER.format(root=ROOT, lib=lib, tests=os.path.join(HERE, "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
