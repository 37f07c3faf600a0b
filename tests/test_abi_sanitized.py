"""The host ABI checks again, against a build whose argument-validation layer
is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only; no GPU, nothing is launched).

Every check of tests/test_abi_host.py runs in a child process with the
sanitizer runtime preloaded and SVGEAR_LIB naming the instrumented library;
any out-of-bounds access, use of freed memory or undefined behaviour in the
validation code aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_checks_pass_under_asan_and_ubsan():
    from sparse_attention_video_means_amd import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=runtime, SVGEAR_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import ctypes, sys; from sparse_attention_video_means_amd import svgear; "
             "svgear.lib(); maps = open('/proc/self/maps').read(); "
             "sys.exit(0 if hasattr(ctypes.CDLL(None), '__asan_init') and "
             "'libsvgear_san' in maps else 3)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, f"instrumented library not in effect:\n{r.stdout[-3000:]}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0 and "passed" in r.stdout, r.stdout[-6000:]
