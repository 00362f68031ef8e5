"""Build libwmtp_hostsan.so: libwmtp with its host code (the C ABI's argument
checks, planning and launch set-up) instrumented by AddressSanitizer and
UndefinedBehaviorSanitizer, for the CPU tests of the C ABI.  Device code is
compiled as in the regular build (sanitizers apply to the host pass only: each
sanitizer flag is handed to the host compiler alone).

    python -m long_context_decode_attention_amd.hostsan

Load it by starting Python with the clang ASan runtime preloaded
(LD_PRELOAD=<runtime()>, ASAN_OPTIONS=detect_leaks=0: the interpreter itself is
not instrumented) and WMTP_LIBRARY=<path>; tests/test_abi_hostsan.py does that.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

from long_context_decode_attention_amd import build as B

LIB = os.path.join(B.HERE, "libwmtp_hostsan.so")

HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def runtime() -> str:
    """The clang ASan runtime that matches hipcc's compiler."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(B.hipcc())))
    hits = sorted(glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang ASan runtime not found next to hipcc")
    return hits[-1]


def build() -> str:
    tmp = LIB + ".tmp"
    res = subprocess.run(B.command(tmp, HOST_SANITIZE), capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libwmtp_hostsan.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    print(runtime())
