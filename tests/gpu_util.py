"""Helpers of the GPU tests: device copies of synthetic inputs, with row
strides, pointer offsets and gap sentinels kept, and bitwise comparison."""
from __future__ import annotations

import hashlib
import sys

import numpy as np

import synth


def say(*a):
    """Name the case before a GPU step (flushed, so a failing run still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def torch():
    import torch as _t
    return _t


def to_device_strided(values: np.ndarray, ld: int, offset: int = 0,
                      gap_bits: int = synth.GAP_IN_BITS):
    """A (rows, cols) float32 CUDA view with row stride ld, starting `offset`
    elements into a buffer whose other elements hold `gap_bits`."""
    t = torch()
    rows, cols = values.shape
    total = offset + max(rows, 1) * ld
    flat = np.empty(total, np.float32)
    flat.view(np.uint32)[:] = np.uint32(gap_bits)
    if rows and cols:
        idx = offset + np.arange(rows)[:, None] * ld + np.arange(cols)[None, :]
        flat[idx] = values
    dflat = t.from_numpy(flat).cuda()
    return t.as_strided(dflat, (rows, cols), (ld, 1), offset), dflat


def to_host(view) -> np.ndarray:
    return view.detach().cpu().numpy()


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def sha256(a) -> str:
    return hashlib.sha256(bits(a).tobytes()).hexdigest()


def assert_same_bits(got, want, what: str):
    g, w = bits(got).ravel(), bits(want).ravel()
    assert g.shape == w.shape, f"{what}: shapes {g.shape} vs {w.shape}"
    if not np.array_equal(g, w):
        bad = np.nonzero(g != w)[0]
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} of {g.size} outputs differ; first at flat "
                             f"index {i}: got {g[i]:08x} want {w[i]:08x}")


# Hash lines of the full-size parity tests: (workload, mode, GPU digest,
# oracle digest, stored digest), printed at the end of the session.
HASH_LINES: list[tuple[str, str, str, str, str]] = []


def record_hashes(workload: str, mode: str, gpu: str, orc: str, stored: str):
    HASH_LINES.append((workload, mode, gpu, orc, stored))
    say(f"sha256 {workload} {mode}: gpu {gpu[:16]} oracle {orc[:16]} stored {stored[:16]}")
