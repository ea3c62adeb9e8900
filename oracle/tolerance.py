"""The accuracy check of fast mode under a stated tolerance (mode 2):
TEST INFRASTRUCTURE, like the rest of this package.

Mode 2 sums each output's products in an order that is not fixed (k split
among waves, four products per matrix-core instruction), so it has no single
correct bit pattern.  What it promises is a bound on the error against the
exact sum, the accuracy bound of "Matrix product and convolution kernels",
section "Fast mode" (k * u * sum |a*b| for sequential summation, u = 2^-24,
plus 1e-30 for subnormals), taken in the form the dotLLM pull request "F32
outer-product tiled GEMM kernel for prefill", section "Tests", checks its
reordered vector path with (4e-6 * sqrt(K), for unit operands), scaled by the
size of the terms:

    |c - r| <= 4e-6 * sqrt(K) * S + 1e-30,

r the exact sum of the output's K products and S the sum of their absolute
values, both computed here in float64 (a float64 sum of binary32 products is
within K * 2^-53 * S of the real sum, far below the bound).  A non-finite
result must have the class of the exact-mode result (the oracle's): NaN for
NaN, the same infinity for an infinity; a finite exact result needs a finite
c.  (The inputs checked here never come near the binary32 overflow
threshold, where a reordered sum could overflow while the sequential one
does not, or the reverse.)
"""
from __future__ import annotations

import math

import numpy as np


def bound(K: int, S: np.ndarray) -> np.ndarray:
    return 4e-6 * math.sqrt(max(K, 1)) * S + 1e-30


def _check(got: np.ndarray, exact: np.ndarray, r: np.ndarray, S: np.ndarray, K: int) -> dict:
    got = np.asarray(got, np.float32)
    exact = np.asarray(exact, np.float32)
    assert got.shape == exact.shape == r.shape == S.shape
    with np.errstate(invalid="ignore"):
        g64 = got.astype(np.float64)
    e_nan, g_nan = np.isnan(exact), np.isnan(got)
    e_inf, g_inf = np.isinf(exact), np.isinf(got)
    finite = ~(e_nan | e_inf)
    class_bad = (e_nan != g_nan) | (e_inf & ~(g_inf & (np.sign(g64) == np.sign(exact)))) | \
                (finite & ~np.isfinite(got))
    tol = bound(K, S)
    both = finite & np.isfinite(got)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.where(both, np.abs(g64 - r), 0.0)
        ratio = np.where(both, err / tol, 0.0)
    over = both & (err > tol)
    return {"outputs": int(got.size), "class_mismatches": int(class_bad.sum()),
            "over_bound": int(over.sum()), "worst_ratio": float(ratio.max()) if ratio.size else 0.0,
            "ok": bool(not class_bad.any() and not over.any())}


def check_gemm(A: np.ndarray, B: np.ndarray, got: np.ndarray, exact: np.ndarray) -> dict:
    """A (m x k) times B (k x n), float32 views; got and exact (m x n)."""
    with np.errstate(invalid="ignore", over="ignore"):  # a signalling NaN input widens to a quiet one
        A64 = np.asarray(A, np.float64)
        B64 = np.asarray(B, np.float64)
        r = A64 @ B64
        S = np.abs(A64) @ np.abs(B64)
    return _check(got, exact, r, S, A.shape[1])


def check_conv(x: np.ndarray, w: np.ndarray, got: np.ndarray, exact: np.ndarray, groups: int = 1,
               stride=(1, 1), pad=(0, 0, 0, 0), dil=(1, 1)) -> dict:
    """NCHW convolution, pad = (top, left, bottom, right); r and S by float64
    convolutions of x, w and of |x|, |w| (padding taps are products with +0)."""
    import torch
    import torch.nn.functional as F

    def conv(a, b):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float64))
        t = F.pad(t, (pad[1], pad[3], pad[0], pad[2]))
        return F.conv2d(t, torch.from_numpy(np.ascontiguousarray(b, np.float64)), stride=stride,
                        dilation=dil, groups=groups).numpy()

    with np.errstate(invalid="ignore", over="ignore"):
        r = conv(x, w)
        S = conv(np.abs(x.astype(np.float64)), np.abs(w.astype(np.float64)))
    K = (x.shape[1] // groups) * w.shape[2] * w.shape[3]
    return _check(got, exact, r, S, K)
