"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer: the host code of
focus_api.hip (argument validation, workspace carving, size queries) is rebuilt with both
sanitizers and tests/test_abi.py runs against it in a child interpreter with the sanitizer
runtime preloaded. Every call there is refused on the host before any device work, so this
runs on a machine without a GPU; any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT


def test_abi_checks_run_clean_under_host_sanitizers():
    from learned_centroid_gated_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = B.build_sanitized()
    env = dict(os.environ)
    env.update(FOCUS_LIB_PATH=lib, LD_PRELOAD=B.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
