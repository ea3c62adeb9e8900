"""GPU parity of the depthwise kernel (Cin/G = 1, any channel multiplier)
against the CPU oracle's direct convolution, bit for bit, exact and fast.

The depthwise kernel computes the convolution expression of "Exact mode",
section "Convolution", directly; so does the oracle.  Cases: random
depthwise shapes with special values (multipliers 1-3, windows 1x1 to 7x7
including the run-time window path, strides, dilations, asymmetric pads,
batch), planes narrower and wider than a wave, padding wider than the
window, and the 15 depthwise convolutions of MobileNetV3-large at batch 1
and 8 in full; the same shapes through the generic implicit-GEMM variants
give the same bits.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import oracle
import synth
from gpu_util import assert_same_bits, say, sha256, to_host, torch

pytestmark = pytest.mark.gpu
MODES = (og.EXACT, og.FAST)


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def auto_variant():
    og.set_variant(0)
    yield
    og.set_variant(0)


def _gpu(x, w, s, mode):
    t = torch()
    y = og.conv2d(t.from_numpy(x).cuda(), t.from_numpy(w).cuda(), stride=s.stride, pad=s.pad,
                  dil=s.dil, groups=s.groups, mode=mode)
    return to_host(y)


def _oracle(orc, x, w, s, mode):
    return orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)


def _specials(a, rng, frac):
    a = a.copy()
    synth.inject_specials(a.reshape(a.shape[0], -1), frac, int(rng.integers(1 << 30)))
    return a


def _random_depthwise(rng, count):
    shapes = []
    while len(shapes) < count:
        C = int(rng.integers(1, 41))
        mult = int(rng.choice([1, 1, 1, 2, 3]))
        KH, KW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        st = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dl = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        pad = tuple(int(p) for p in rng.integers(0, 5, size=4))
        if H + pad[0] + pad[2] - dl[0] * (KH - 1) - 1 < 0:
            continue
        if W + pad[1] + pad[3] - dl[1] * (KW - 1) - 1 < 0:
            continue
        shapes.append(synth.ConvShape(f"dw{len(shapes)}", int(rng.integers(1, 4)), C, H, W,
                                      C * mult, KH, KW, st, pad, dl, C))
    return shapes


@pytest.mark.parametrize("mode", MODES)
def test_random_depthwise_shapes(orc, mode):
    rng = np.random.default_rng(600 + mode)
    for s in _random_depthwise(rng, 80):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _specials(x, rng, 0.01)
        w = _specials(w, rng, 0.02)
        say(f"depthwise {s} mode {mode}")
        assert_same_bits(_gpu(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


def test_plane_edges(orc):
    """Planes of exactly one wave, one pixel more, a 1x1 plane, padding wider
    than the window, and a plane of many waves with a ragged last one."""
    shapes = [synth.ConvShape("one_wave", 2, 3, 8, 8, 3, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 3),
              synth.ConvShape("wave_plus_1", 1, 5, 5, 13, 10, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 5),
              synth.ConvShape("pixel", 3, 7, 1, 1, 7, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 7),
              synth.ConvShape("wide_pad", 1, 4, 3, 2, 8, 3, 3, (1, 1), (4, 3, 4, 3), (1, 1), 4),
              synth.ConvShape("many", 1, 2, 37, 53, 2, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 2),
              synth.ConvShape("strided", 2, 6, 31, 29, 6, 5, 5, (2, 3), (2, 1, 0, 2), (1, 2), 6),
              synth.ConvShape("k7", 1, 3, 20, 20, 6, 7, 7, (1, 1), (3, 3, 3, 3), (1, 1), 3)]
    rng = np.random.default_rng(650)
    for s in shapes:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _specials(x, rng, 0.02)
        for mode in MODES:
            say(f"depthwise edge {s} mode {mode}")
            assert_same_bits(_gpu(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


def test_several_outputs_per_lane(orc):
    """Stride-1 3x3 launches with many planes run 4 or 2 outputs per lane
    (2400 planes of 255 pixels: four per lane, the last wave of a plane
    ragged; 1400 planes of 130 pixels: two per lane)."""
    rng = np.random.default_rng(660)
    for s in (synth.ConvShape("p4", 4, 600, 15, 17, 600, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 600),
              synth.ConvShape("p2", 2, 700, 10, 13, 700, 3, 3, (1, 1), (1, 0, 1, 2), (1, 1), 700)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _specials(x, rng, 0.001)
        for mode in MODES:
            say(f"depthwise several per lane {s} mode {mode}")
            assert_same_bits(_gpu(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


def test_band_form(orc):
    """Strided 3x3 and 5x5 windows on planes 28+ wide with enough planes run
    the band form (input rows staged in LDS): ragged last bands, padding on
    every side, dilation, a multiplier of 2."""
    rng = np.random.default_rng(670)
    for s in (synth.ConvShape("b3s2", 8, 64, 112, 112, 64, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 64),
              synth.ConvShape("b5s1", 8, 120, 28, 28, 120, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 120),
              synth.ConvShape("b5s2", 8, 72, 57, 58, 72, 5, 5, (2, 2), (2, 1, 3, 2), (1, 1), 72),
              synth.ConvShape("b3d2", 4, 300, 30, 60, 600, 3, 3, (1, 2), (2, 2, 2, 2), (2, 2), 300),
              synth.ConvShape("b5big", 2, 600, 40, 61, 600, 5, 5, (1, 1), (0, 4, 1, 0), (1, 1), 600)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _specials(x, rng, 0.0005)
        w = _specials(w, rng, 0.002)
        for mode in MODES:
            say(f"depthwise band {s} mode {mode}")
            assert_same_bits(_gpu(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


def test_padding_tap_meets_infinite_weight():
    """A depthwise output whose only non-padding tap is finite still turns NaN
    when an infinite weight meets a padding tap (padding taps are real products)."""
    s = synth.ConvShape("w8dw", 1, 2, 1, 1, 2, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 2)
    x = np.array([[[[2.0]], [[3.0]]]], np.float32)
    w = np.ones((2, 1, 3, 3), np.float32)
    w[0, 0, 0, 0] = np.inf
    for mode in MODES:
        y = _gpu(x, w, s, mode).view(np.uint32).ravel()
        assert y[0] == 0x7FC00000 and y[1] == np.float32(3.0).view(np.uint32)


@pytest.mark.parametrize("batch", [1, 8])
def test_mobilenetv3_depthwise_layers(orc, batch):
    """The 15 depthwise layers of MobileNetV3-large, every output of both modes."""
    for i, s in enumerate(synth.mobilenetv3_large_depthwise(batch)):
        x, w = synth.conv_inputs(s, synth.seed_for(6, 100 * batch + i))
        for mode in MODES:
            say(f"mobilenetv3 {s} mode {mode}")
            got = _gpu(x, w, s, mode)
            want = _oracle(orc, x, w, s, mode)
            assert sha256(got) == sha256(want), f"{s} mode {mode}"


@pytest.mark.parametrize("variant", [1, 3, 6, 10, 14, 17, 18])
def test_generic_variants_agree(orc, variant):
    """Forced implicit-GEMM variants (and 18, the depthwise kernel) give the same bits."""
    og.set_variant(variant)
    rng = np.random.default_rng(700)
    for s in (synth.ConvShape("g3", 2, 12, 15, 9, 24, 3, 3, (1, 2), (1, 0, 2, 1), (2, 1), 12),
              synth.ConvShape("g5", 1, 9, 11, 12, 9, 5, 5, (2, 2), (2, 2, 2, 2), (1, 1), 9)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        for mode in MODES:
            say(f"depthwise variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"variant {variant} {s} mode {mode}")
