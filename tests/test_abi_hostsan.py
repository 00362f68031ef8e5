"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only: the sanitizers instrument the host pass of the library build, and
nothing here launches a kernel).  Builds libwmtp_hostsan.so when it is missing
or older than its sources, then runs the CPU tests of the C ABI
(test_abi_cpu.py: symbol table, every argument check, the planner sweep over
extreme sizes) in a child process that preloads the clang ASan runtime and
loads the sanitized library through WMTP_LIBRARY.  Any sanitizer report aborts
the child, and the test fails with its output."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_decode_attention_amd")


def _stale(lib):
    if not os.path.exists(lib):
        return True
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + [os.path.join(ROOT, "include", "wmtp.h")]
    return max(os.path.getmtime(f) for f in srcs) > os.path.getmtime(lib)


def test_abi_under_host_sanitizers():
    hostsan = pytest.importorskip("long_context_decode_attention_amd.hostsan")
    try:
        hostsan.B.hipcc()
        runtime = hostsan.runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale(hostsan.LIB):
        hostsan.build()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "WMTP_LIBRARY": hostsan.LIB,
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
