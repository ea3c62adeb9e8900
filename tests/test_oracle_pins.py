"""The CPU oracle against its pins (hand-worked cases, closed forms, IEEE
arithmetic on exact rationals, invariants, library routines)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_selftest_runs_at_load(orc):
    assert orc.L.ogref_selftest() == 0


def test_invalid_arguments_rejected(orc):
    import numpy as np
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 4), np.float32)
    with pytest.raises(ValueError):
        orc.gemm(A, B, 7)
    x = np.ones((1, 4, 5, 5), np.float32)
    w = np.ones((2, 2, 3, 3), np.float32)
    with pytest.raises(ValueError):  # Cout not a multiple of the 3 groups is caught in C
        orc.conv2d(np.ones((1, 3, 5, 5), np.float32), np.ones((2, 1, 3, 3), np.float32), 0,
                   groups=3)
    with pytest.raises(ValueError):  # window larger than the padded input
        orc.conv2d(np.ones((1, 2, 2, 2), np.float32), np.ones((1, 2, 3, 3), np.float32), 0)
    assert orc.conv2d(x, w, 0, groups=2).shape == (1, 2, 3, 3)


def test_thread_count_does_not_change_bits(orc):
    """The oracle's OpenMP split is over outputs only: 1 thread and all threads
    give the same bits, both modes, product and convolution."""
    import numpy as np
    rng = np.random.default_rng(11)
    A = rng.standard_normal((37, 300)).astype(np.float32)
    B = rng.standard_normal((300, 41)).astype(np.float32)
    x = rng.standard_normal((2, 6, 9, 8)).astype(np.float32)
    w = rng.standard_normal((4, 3, 3, 3)).astype(np.float32)
    full = orc.num_threads()
    try:
        res = {}
        for n in (1, max(2, full)):
            assert orc.set_num_threads(n) == n
            res[n] = [orc.gemm(A, B, m) for m in (0, 1)] + [
                orc.gemm(A, B, m, rowwise=True) for m in (0, 1)] + [
                orc.conv2d(x, w, m, groups=2, stride=(2, 1), pad=(1, 0, 2, 1)) for m in (0, 1)]
        for a, b in zip(res[1], res[max(2, full)]):
            pins.assert_bits_equal(a, b, "1 thread vs all threads")
    finally:
        orc.set_num_threads(full)
