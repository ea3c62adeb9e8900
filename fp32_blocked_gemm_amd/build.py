"""Build libog.so in-tree with hipcc for gfx950.

The floating-point flags are part of the contract: no contraction of a*b+c
(-ffp-contract=off), fp32 denormals kept (-fno-gpu-flush-denormals-to-zero),
no packed-fp32 VALU forms, and MFMA results in ordinary VGPRs so that exact
mode's separately rounded adds read them directly.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libog.so")
SOURCES = [os.path.join(CSRC, "og_api.hip")]
HEADERS = [os.path.join(CSRC, "og_kernels.hpp"), os.path.join(INCLUDE, "og.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
]


def _digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile libog.so (always; a few minutes).

    hipcc reads the sources once for the device code and again for the host
    code; a source edited in between would give a library whose host side
    launches kernels its device code does not have.  The sources are hashed
    before and after, and a library built from sources that changed meanwhile
    is rejected.
    """
    before = _digest()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that note is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    if _digest() != before:
        os.remove(LIB + ".tmp")
        raise RuntimeError("the sources changed during the build; build again")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
