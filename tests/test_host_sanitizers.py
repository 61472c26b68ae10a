"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds _build/libgdpa_asan.so (gdpa_api.cpp compiled with host-only sanitizer
flags, the kernels unchanged) and runs the CPU-only boundary tests against it in a
child process that preloads clang's sanitizer runtime.  No GPU call is made: every
case of those tests fails validation before any HIP call, or only reads the
exported table of entry points.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from context_cross_attention_amd import build  # noqa: E402


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_abi_checks_under_asan_and_ubsan():
    lib = build.build_sanitized(verbose=False)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms, "the C ABI is not instrumented"
    rt = build.san_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, GDPA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = ("import sys, context_cross_attention_amd as cca, pytest; "
            f"assert cca.LIB_PATH == {lib!r}; "
            "sys.exit(pytest.main(['-x', '-q', '-m', 'not gpu', '-p', 'no:cacheprovider', "
            "'tests/test_abi.py', 'tests/test_binding_checks.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
