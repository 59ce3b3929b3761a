"""The C ABI's host code under AddressSanitizer.

CPU only.  The library is built again with its host code instrumented
(argument validation, workspace sizing, dispatch; sanitizers are never used in
device code), and the ABI cases of test_abi.py run against that build in a
child process that preloads the sanitizer runtime.  Every case fails
validation before anything is enqueued, so no GPU is needed; an out-of-bounds
or use-after-free access in the host code would abort the child with a
sanitizer report.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cases_under_address_sanitizer(tmp_path):
    from query_guided_kv_amd import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_asan(str(tmp_path / "asan"))
    env = dict(os.environ, LD_PRELOAD=runtime, KVSEL_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
