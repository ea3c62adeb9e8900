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
OBJDIR = os.path.join(HERE, "_build")
API = os.path.join(CSRC, "og_api.hip")
UNITS = os.path.join(CSRC, "og_units.hip")
N_UNITS = 17  # kernel groups of og_units.hip, compiled in parallel
SOURCES = [API, UNITS]
HEADERS = [os.path.join(CSRC, "og_kernels.hpp"), os.path.join(CSRC, "og_launch.hpp"),
           os.path.join(INCLUDE, "og.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
]
# the host pass does not know the packed-fp32 target feature; that note is harmless
NOISE = "is not a recognized feature for this target"


def _digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _jobs() -> int:
    n = os.cpu_count() or 4
    try:
        n = min(n, int(os.environ.get("MAX_JOBS", n)))
    except ValueError:
        pass
    return max(1, min(n, 16))


def build(verbose: bool = False) -> str:
    """Compile libog.so (always): og_api.hip and each kernel group of
    og_units.hip as separate objects, compiled in parallel, then linked.

    hipcc reads the sources once for the device code and again for the host
    code; a source edited in between would give a library whose host side
    launches kernels its device code does not have.  The sources are hashed
    before and after, and a library built from sources that changed meanwhile
    is rejected.
    """
    before = _digest()
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = [(API, [], os.path.join(OBJDIR, "og_api.o"))]
    jobs += [(UNITS, [f"-DOG_UNIT={u}"], os.path.join(OBJDIR, f"og_unit{u}.o"))
             for u in range(1, N_UNITS + 1)]
    cmds = [[HIPCC, *FLAGS, *inc, *defs, "-c", src, "-o", obj] for src, defs, obj in jobs]
    pending, running, msgs, failed = list(cmds), [], [], []
    limit = _jobs()
    while pending or running:
        while pending and len(running) < limit:
            cmd = pending.pop(0)
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.STDOUT, text=True)))
        cmd, proc = running.pop(0)
        out, _ = proc.communicate()
        lines = [l for l in out.splitlines() if NOISE not in l]
        msgs += lines
        if proc.returncode != 0:
            failed.append(cmd[-1])
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}:\n" + "\n".join(msgs))
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[obj for *_, obj in jobs],
            "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    msgs += [l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l]
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
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
