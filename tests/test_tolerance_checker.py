"""The mode-2 accuracy check (oracle/tolerance.py) against things other than
itself: it accepts the oracle's exact and fast results (sequential sums: their
worst-case error gamma_K * S lies inside 4e-6 * sqrt(K) * S up to K of about
4500, and their typical error, near sqrt(K) * 2^-24 * S, far inside), rejects
a result moved just past the bound, a dropped term and every class mismatch,
and its reference sum equals numpy's int64 product on integer inputs."""
import math

import numpy as np
import pytest

import oracle
from oracle import tolerance

EXACT, FAST = 0, 1


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _specials(rng, a, frac):
    a = a.copy()
    flat = a.reshape(-1)
    pos = rng.choice(flat.size, size=max(1, int(frac * flat.size)), replace=False)
    flat[pos] = rng.choice(np.array([np.nan, np.inf, -np.inf, 1e-40, -0.0], np.float32), pos.size)
    return a


@pytest.mark.parametrize("m,n,k", [(7, 9, 1), (13, 17, 64), (5, 33, 1531), (3, 40, 4096)])
def test_accepts_exact_and_fast_sequential_sums(orc, m, n, k):
    rng = np.random.default_rng(m * n + k)
    for A, B in ((rng.standard_normal((m, k)).astype(np.float32),
                  rng.standard_normal((k, n)).astype(np.float32)),
                 (rng.uniform(0, 1, (m, k)).astype(np.float32),        # same-sign terms:
                  rng.uniform(0, 1, (k, n)).astype(np.float32)),       # the largest error
                 (_specials(rng, rng.standard_normal((m, k)).astype(np.float32), 0.02),
                  _specials(rng, rng.standard_normal((k, n)).astype(np.float32), 0.02))):
        exact = orc.gemm(A, B, EXACT)
        for mode in (EXACT, FAST):
            rep = tolerance.check_gemm(A, B, orc.gemm(A, B, mode), exact)
            assert rep["ok"], (mode, rep)


def test_accepts_convolutions(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 6, 9, 8)).astype(np.float32)
    w = rng.standard_normal((4, 3, 3, 3)).astype(np.float32)
    kw = dict(groups=2, stride=(2, 1), pad=(1, 0, 2, 1), dil=(1, 2))
    exact = orc.conv2d(x, w, EXACT, **kw)
    for mode in (EXACT, FAST):
        rep = tolerance.check_conv(x, w, orc.conv2d(x, w, mode, **kw), exact, **kw)
        assert rep["ok"], rep


def test_rejects_a_result_just_past_the_bound(orc):
    rng = np.random.default_rng(5)
    A = rng.standard_normal((4, 300)).astype(np.float32)
    B = rng.standard_normal((300, 6)).astype(np.float32)
    exact = orc.gemm(A, B, EXACT)
    r = A.astype(np.float64) @ B.astype(np.float64)
    S = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    tol = tolerance.bound(300, S)
    for scale, ok in ((1.02, False), (0.5, True)):
        got = exact.copy()
        c = np.float32(r[2, 3] + scale * tol[2, 3])
        while not ok and abs(float(c) - r[2, 3]) <= tol[2, 3]:  # step just past the bound
            c = np.nextafter(c, np.float32(np.inf))
        got[2, 3] = c
        rep = tolerance.check_gemm(A, B, got, exact)
        assert rep["ok"] == ok, (scale, rep)
        if not ok:
            assert rep["over_bound"] == 1


def test_rejects_a_dropped_term(orc):
    rng = np.random.default_rng(6)
    A = rng.standard_normal((3, 500)).astype(np.float32)
    B = rng.standard_normal((500, 4)).astype(np.float32)
    exact = orc.gemm(A, B, EXACT)
    A2 = A.copy()
    A2[1, 250] = 0.0  # one product left out of row 1
    got = orc.gemm(A2, B, FAST)
    rep = tolerance.check_gemm(A, B, got, exact)
    assert not rep["ok"] and rep["over_bound"] >= 1


def test_rejects_class_mismatches(orc):
    rng = np.random.default_rng(7)
    A = rng.standard_normal((2, 8)).astype(np.float32)
    B = rng.standard_normal((8, 3)).astype(np.float32)
    A[0, 3] = np.inf   # row 0: +-inf or NaN
    A[1, 2] = np.nan   # row 1: NaN
    exact = orc.gemm(A, B, EXACT)
    assert tolerance.check_gemm(A, B, exact.copy(), exact)["ok"]
    for (i, j, v) in ((1, 0, 1.0), (0, 1, np.nan), (0, 1, 1e30)):
        got = exact.copy()
        got[i, j] = v
        assert not tolerance.check_gemm(A, B, got, exact)["ok"], (i, j, v)
    got = exact.copy()
    j = int(np.nonzero(np.isinf(exact[0]))[0][0])
    got[0, j] = -exact[0, j]  # the other infinity
    assert not tolerance.check_gemm(A, B, got, exact)["ok"]
    # a finite exact result with an infinite answer
    A3 = rng.standard_normal((2, 8)).astype(np.float32)
    e3 = orc.gemm(A3, B, EXACT)
    g3 = e3.copy()
    g3[1, 1] = np.inf
    assert not tolerance.check_gemm(A3, B, g3, e3)["ok"]


def test_reference_sum_is_the_integer_product():
    """On small integers the float64 reference is exact: numpy's int64 product."""
    rng = np.random.default_rng(8)
    Ai = rng.integers(-8, 9, (5, 70))
    Bi = rng.integers(-8, 9, (70, 6))
    A, B = Ai.astype(np.float32), Bi.astype(np.float32)
    want = (Ai @ Bi).astype(np.float32)
    rep = tolerance.check_gemm(A, B, want, want)
    assert rep["ok"] and rep["worst_ratio"] == 0.0
    off = want.copy()
    off[0, 0] += 1.0  # a unit error on sums of at most 70 * 64: past 4e-6 * sqrt(70) * S
    assert not tolerance.check_gemm(A, B, off, want)["ok"]


def test_bound_formula():
    assert tolerance.bound(100, np.array([1.0]))[0] == pytest.approx(4e-5 + 1e-30)
    assert tolerance.bound(0, np.array([0.0]))[0] == 1e-30
    assert tolerance.bound(4096, np.array([2.0]))[0] == pytest.approx(4e-6 * 64 * 2)
    assert math.isclose(tolerance.bound(4608, np.array([1.0]))[0], 4e-6 * math.sqrt(4608))
