"""The host side of the library (argument validation, the batched planner,
the workspace carve-up) under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with sanitized host code (device code as usual) and
the CPU ABI suite, which includes a fuzz test of the planner, runs against it
in a child process with the ASan runtime preloaded.  No kernel is launched.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_asan_and_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set; the ASan runtime must come first")
    if not shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc")
    from newton_schulz_matrix_muon_amd import build

    lib = build.build_sanitized()
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=rt,
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        MUON_LIBRARY=lib,
    )
    r = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
         "-p", "no:cacheprovider"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600,
    )
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
