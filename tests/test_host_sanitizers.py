"""The C-ABI host code (argument checks, permutations, the normal quantile) under AddressSanitizer
and UndefinedBehaviorSanitizer: the library's host sources are rebuilt with both sanitizers on the
host pass (build.build_host_sanitized) and the whole CPU tier of the ABI (test_abi_cpu.py) runs
against that build in a child process with the sanitizer runtime preloaded.  Any report aborts
the child (halt_on_error), so the test fails on the first finding."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tier_clean_under_asan_and_ubsan():
    from dynamic_block_sparse_gilbert_amd import build
    rt = build.asan_runtime()
    if not rt:
        pytest.skip("no shared AddressSanitizer runtime next to hipcc")
    lib = build.build_host_sanitized()
    with open(lib, "rb") as f:
        blob = f.read()
    assert b"__asan_report" in blob and b"__ubsan_handle" in blob    # instrumented
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, DBS_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-s",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
