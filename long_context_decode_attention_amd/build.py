"""Build libwmtp.so (HIP, gfx950) in place, next to this file.

    python -m long_context_decode_attention_amd.build

Every HIP source under csrc/ is compiled for gfx950 only.  Packed fp32 VALU
instructions are switched off for the device code (`-packed-fp32-ops`); the
host pass warns that it does not know that feature, which is harmless.  Device
code is built with `-fno-honor-nans`: the kernels never rely on NaN semantics
(absent keys are masked with selects and integer masks, not NaN tests), and it
spares the max reductions of the softmax a canonicalising instruction per input.
Host code keeps full IEEE semantics, so argument checks still see NaN.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwmtp.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwmtp.so)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def command(out: str = LIB, extra: list | None = None) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xarch_device", "-fno-honor-nans",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *(extra or []), *sources(), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libwmtp.so; returns its path.  Always rebuilds."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libwmtp.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
