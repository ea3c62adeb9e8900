"""Pins of the oracle's convolution epilogue ("Convolution (fast mode)",
sections "Tiles and chunks" and "Single-column products": bias, then the
activation, then the residual, on the finished sum).

The order is pinned by hand-worked values that every other order gets wrong;
the bias step by an identity with the oracle's own (separately pinned)
convolution: a bias equals one more input channel of ones whose 1x1 weight is
the bias, summed last; the ReLU and residual steps by numpy's IEEE float32
arithmetic and by integer closed forms; special values by IEEE rules.
"""
import numpy as np
import pytest

import oracle

CANON = 0x7FC00000


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _t(v):
    return np.array(v, np.float32).reshape(1, -1, 1, 1)


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_order_bias_relu_residual(orc):
    """y = -3, bias 1, residual 5: bias-ReLU-residual gives 5; residual before
    ReLU gives 3, ReLU before bias gives 6, no ReLU gives 3."""
    got = orc.conv_epilogue(_t([-3.0]), np.float32([1.0]), 1, _t([5.0]))
    assert got.ravel()[0] == 5.0
    # a positive sum passes ReLU unchanged: 2 + 1 = 3, + 5 = 8
    got = orc.conv_epilogue(_t([2.0]), np.float32([1.0]), 1, _t([5.0]))
    assert got.ravel()[0] == 8.0
    # the bias is per output channel, the residual per position
    y = np.arange(12, dtype=np.float32).reshape(1, 3, 2, 2) - 6.0
    b = np.float32([10.0, -20.0, 0.5])
    r = np.full_like(y, 0.25)
    want = np.maximum(y + b.reshape(1, 3, 1, 1), 0) + r
    assert np.array_equal(orc.conv_epilogue(y, b, 1, r), want)


def test_signed_zero_and_nan(orc):
    """ReLU maps -0 and negatives to +0 and keeps a NaN (stored as the
    canonical NaN); without ReLU -0 survives; inf + -inf residual is NaN."""
    y = np.array([-0.0, -1e-45, np.nan, np.inf, -np.inf, 0.0], np.float32).reshape(1, 6, 1, 1)
    y.view(np.uint32).ravel()[2] = 0xFFC12345  # a negative NaN with a payload
    got = _bits(orc.conv_epilogue(y, None, 1, None)).ravel()
    assert list(got) == [0, 0, CANON, 0x7F800000, 0, 0]
    got = _bits(orc.conv_epilogue(y, None, 0, None)).ravel()
    assert list(got) == [0x80000000, 0x80000001, CANON, 0x7F800000, 0xFF800000, 0]
    # -0 + -0 bias stays -0 without ReLU, +0 with it
    got = _bits(orc.conv_epilogue(_t([-0.0]), np.float32([-0.0]), 0, None)).ravel()
    assert got[0] == 0x80000000
    got = _bits(orc.conv_epilogue(_t([-0.0]), np.float32([-0.0]), 1, None)).ravel()
    assert got[0] == 0
    # inf (after ReLU) + -inf residual: invalid, canonical NaN
    got = _bits(orc.conv_epilogue(_t([np.inf]), None, 1, _t([-np.inf]))).ravel()
    assert got[0] == CANON
    # a NaN bias turns every output of its channel to the canonical NaN, ReLU or not
    got = _bits(orc.conv_epilogue(_t([1.0, -2.0]), np.float32([np.nan, 0.0]), 1, None)).ravel()
    assert list(got) == [CANON, 0]


def test_integer_closed_form(orc):
    """Small integers add exactly: max(y + b, 0) + r in int64."""
    rng = np.random.default_rng(3)
    yi = rng.integers(-1000, 1000, size=(2, 5, 3, 4))
    bi = rng.integers(-500, 500, size=5)
    ri = rng.integers(-1000, 1000, size=yi.shape)
    got = orc.conv_epilogue(yi.astype(np.float32), bi.astype(np.float32), 1,
                            ri.astype(np.float32))
    want = np.maximum(yi + bi.reshape(1, 5, 1, 1), 0) + ri
    assert np.array_equal(got.astype(np.int64), want)
    got = orc.conv_epilogue(yi.astype(np.float32), bi.astype(np.float32), 0, None)
    assert np.array_equal(got.astype(np.int64), yi + bi.reshape(1, 5, 1, 1))


def test_rounding_matches_float32_adds(orc):
    """Each add rounds once to float32, as numpy's float32 add does."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((3, 7, 5, 6)).astype(np.float32)
    b = rng.standard_normal(7).astype(np.float32) * np.float32(1e3)
    r = rng.standard_normal(y.shape).astype(np.float32) * np.float32(1e-3)
    v = y + b.reshape(1, 7, 1, 1)
    want = np.where(v > 0, v, np.float32(0)) + r
    assert np.array_equal(_bits(orc.conv_epilogue(y, b, 1, r)), _bits(want))
    assert np.array_equal(_bits(orc.conv_epilogue(y, None, 0, r)), _bits(y + r))


@pytest.mark.parametrize("mode", [0, 1])
def test_bias_equals_a_last_channel_of_ones(orc, mode):
    """A 1x1 convolution (no padding) with bias b equals the same convolution
    with one more input channel, all ones, whose weight for output channel oc
    is b[oc]: the extra channel is the last term of each sum, and in both
    modes adding 1 * b rounds once, as the epilogue's s + b does."""
    rng = np.random.default_rng(10 + mode)
    N, Cin, H, W, Cout = 2, 6, 5, 7, 9
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = rng.standard_normal((Cout, Cin, 1, 1)).astype(np.float32)
    b = rng.standard_normal(Cout).astype(np.float32)
    x1 = np.concatenate([x, np.ones((N, 1, H, W), np.float32)], axis=1)
    w1 = np.concatenate([w, b.reshape(Cout, 1, 1, 1)], axis=1)
    want = orc.conv2d(x1, w1, mode)
    got = orc.conv_epilogue(orc.conv2d(x, w, mode), b, 0, None)
    assert np.array_equal(_bits(got), _bits(want))


def test_invalid_activation(orc):
    with pytest.raises(ValueError):
        orc.conv_epilogue(_t([1.0]), None, 2, None)
