"""The full-size workloads of the parity tests: their inputs (from synth),
the oracle's outputs and the SHA-256 of those outputs, per workload and mode.

TEST INFRASTRUCTURE: this module imports the oracle and synth, never the GPU
package.  ``tests/golden/make_full_size_hashes.py`` writes the oracle's
digests to ``tests/golden/full_size_sha256.json``; the GPU parity tests
compare the GPU's outputs with the oracle's element by element and both
digests with the stored one, the way "Exact mode", section "Checking it",
compares every path with the naive definition and keeps hash lines that must
be equal on every machine.

A digest covers a workload's outputs in order (a chain of convolutions: every
layer's output), each as its binary32 bit patterns in C order (a matrix:
its logical m x n elements, not the gaps of a row stride).
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
STORED = os.path.join(HERE, "golden", "full_size_sha256.json")
MODES = {"exact": 0, "fast": 1}

GEMMS = {
    "gemm_256": synth.gemm_square256,
    "gemm_4096_specials": lambda: synth.gemm_4096(True),
    "gemm_4096_clean": lambda: synth.gemm_4096(False),
    "gemm_ragged_specials": lambda: synth.gemm_ragged(True),
    "gemm_ragged_clean": lambda: synth.gemm_ragged(False),
    "gemm_prefill": synth.gemm_prefill,
    "gemm_skinny": synth.gemm_skinny,
}

# name -> (layers, seed of layer i, value distribution)
CONVS = {
    "resnet50_b1": (lambda: synth.resnet50_convs(1), lambda i: synth.seed_for(4, i), "normal"),
    "resnet50_b8": (lambda: synth.resnet50_convs(8), lambda i: synth.seed_for(4, 100 + i),
                    "normal"),
    "grouped_dilated": (lambda: [synth.grouped_dilated()], lambda i: synth.seed_for(5, 0),
                        "uniform"),
    "conv1d_h1": (lambda: [synth.conv1d_h1()], lambda i: synth.seed_for(5, 10), "uniform"),
}


def gemm_case(name: str) -> synth.GemmCase:
    return GEMMS[name]()


def conv_layers(name: str):
    """(shape, x, w) of each convolution of the workload, generated one at a time."""
    layers, seed, dist = CONVS[name]
    for i, s in enumerate(layers()):
        x, w = synth.conv_inputs(s, seed(i), dist)
        yield s, x, w


def oracle_gemm(orc, case: synth.GemmCase, mode: int) -> np.ndarray:
    return orc.gemm(case.A, case.B, mode, rowwise=True)


def oracle_conv(orc, s: synth.ConvShape, x: np.ndarray, w: np.ndarray, mode: int) -> np.ndarray:
    # the im2col route: pinned equal to the direct definition, and much faster
    return orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil,
                      route="im2col")


class Digest:
    """SHA-256 over a sequence of outputs, each as its uint32 bit patterns."""

    def __init__(self):
        self.h = hashlib.sha256()

    def add(self, a: np.ndarray) -> "Digest":
        self.h.update(np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).tobytes())
        return self

    def hex(self) -> str:
        return self.h.hexdigest()


def oracle_digest(orc, name: str, mode: int) -> str:
    d = Digest()
    if name in GEMMS:
        d.add(oracle_gemm(orc, gemm_case(name), mode))
    else:
        for s, x, w in conv_layers(name):
            d.add(oracle_conv(orc, s, x, w, mode))
    return d.hex()


def stored() -> dict:
    with open(STORED) as f:
        return json.load(f)
