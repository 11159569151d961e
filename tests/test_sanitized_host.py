"""The library's host side built with AddressSanitizer and UndefinedBehavior-
Sanitizer (device code unchanged) runs the C-ABI, binding-shape and host
self-test checks, which need no GPU: every argument-validation path, the
layout maps of the permutation kernels run on the host, the XCD deal and the
allocation-free profiler's host checks must run without a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_validation_under_asan_and_ubsan():
    from block_sparse_attention_vsa_amd.build import build, sanitizer_runtime
    lib = build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=sanitizer_runtime(), VSA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import block_sparse_attention_vsa_amd as V; assert V.LIB_PATH.endswith('libvsa_sanitized.so'); "
            "V.vsa_selftest_host(); print('selftest ok')")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "selftest ok" in out, out[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_binding_shapes.py", "tests/test_zz_no_alloc.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in out, out[-3000:]
