"""GPU parity of the fused convolution epilogue ("Convolution (fast mode)",
sections "Tiles and chunks" and "Single-column products": bias, then ReLU,
then the residual, on each finished sum) against the oracle's convolution
followed by the oracle's epilogue, bit for bit, exact and fast.

Every kernel that stores convolution outputs applies the epilogue at its
store: the implicit-GEMM variants 1-20 (forced), the depthwise kernel (one
and several outputs per lane, the band form), the grouped direct kernel, the
single-column products of squeeze-and-excitation layers, and the shapes'
automatic choices.  The residual may be the output itself (read before the
write); bias and residual carry special values.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import oracle
import synth
from gpu_util import assert_same_bits, say, to_host, torch

pytestmark = pytest.mark.gpu
MODES = (og.EXACT, og.FAST)
# (bias, relu, residual, residual is the output)
COMBOS = [(True, False, False, False), (False, True, False, False), (False, False, True, False),
          (True, True, True, False), (True, True, True, True)]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def auto_variant():
    og.set_variant(0)
    yield
    og.set_variant(0)


def _specials(a, rng, frac):
    a = a.copy()
    synth.inject_specials(a.reshape(1 if a.ndim == 1 else a.shape[0], -1), frac,
                          int(rng.integers(1 << 30)))
    return a


def _out_shape(s):
    OH = og.conv2d_out_size(s.H, s.KH, s.stride[0], s.pad[0], s.pad[2], s.dil[0])
    OW = og.conv2d_out_size(s.W, s.KW, s.stride[1], s.pad[1], s.pad[3], s.dil[1])
    return (s.N, s.Cout, OH, OW)


def _check(orc, s, x, w, rng, combos=COMBOS, modes=MODES, special_frac=0.01, tag=""):
    t = torch()
    dx, dw = t.from_numpy(x).cuda(), t.from_numpy(w).cuda()
    shape = _out_shape(s)
    bias = _specials(rng.standard_normal(s.Cout).astype(np.float32), rng, special_frac)
    res = _specials(rng.standard_normal(shape).astype(np.float32), rng, special_frac)
    db, dr = t.from_numpy(bias).cuda(), t.from_numpy(res).cuda()
    for mode in modes:
        sums = orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)
        for use_b, relu, use_r, in_place in combos:
            say(f"epilogue {tag} {s} mode {mode} bias={use_b} relu={relu} res={use_r} "
                f"in_place={in_place}")
            want = orc.conv_epilogue(sums, bias if use_b else None, 1 if relu else 0,
                                     res if use_r else None)
            out = dr.clone() if in_place else None
            r = (out if in_place else dr) if use_r else None
            y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups,
                          mode=mode, out=out, bias=db if use_b else None,
                          act="relu" if relu else None, residual=r)
            assert_same_bits(to_host(y), want, f"{tag} {s} mode {mode} combo "
                             f"{(use_b, relu, use_r, in_place)}")


@pytest.mark.parametrize("variant", list(range(1, 21)))
def test_every_variant(orc, variant):
    """A strided, padded 3x3 convolution and a 1x1 one over several tiles with
    ragged edges, through each forced variant."""
    og.set_variant(variant)
    rng = np.random.default_rng(900 + variant)
    for s in (synth.ConvShape("r3", 2, 12, 15, 11, 37, 3, 3, (1, 2), (1, 0, 2, 1), (1, 1), 1),
              synth.ConvShape("p1", 1, 40, 9, 30, 70, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 1)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _specials(x, rng, 0.002)
        _check(orc, s, x, w, rng, tag=f"variant {variant}")


def test_automatic_choices(orc):
    """Shapes whose automatic choice is a large-tile variant, a chain, or the
    planes and gather forms of the implicit GEMM."""
    rng = np.random.default_rng(950)
    for s in (synth.ConvShape("res3", 2, 64, 28, 28, 128, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 1),
              synth.ConvShape("res1", 4, 256, 14, 14, 256, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 1),
              synth.ConvShape("few", 1, 96, 40, 40, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
              synth.ConvShape("stem", 1, 3, 64, 64, 16, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 1),
              synth.ConvShape("conv1d", 2, 80, 1, 300, 96, 1, 3, (1, 1), (0, 1, 0, 1), (1, 1), 1)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)))
        _check(orc, s, x, w, rng, tag="auto")


def test_depthwise_paths(orc):
    """The depthwise kernel: one output per lane, several per lane (2400
    planes of a stride-1 3x3), and the band form (strided 3x3, 5x5)."""
    rng = np.random.default_rng(960)
    for s in (synth.ConvShape("dw", 2, 24, 19, 23, 48, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 24),
              synth.ConvShape("p4", 4, 600, 15, 17, 600, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 600),
              synth.ConvShape("b3s2", 8, 64, 112, 112, 64, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 64),
              synth.ConvShape("b5s1", 8, 120, 28, 28, 120, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 120)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        _check(orc, s, x, w, rng, special_frac=0.001, tag="depthwise")


def test_grouped_direct_kernel(orc):
    rng = np.random.default_rng(970)
    for s in (synth.ConvShape("g8x8", 2, 64, 20, 18, 64, 3, 3, (2, 2), (2, 2, 2, 2), (2, 2), 8),
              synth.ConvShape("g5", 1, 100, 17, 9, 25, 3, 3, (2, 1), (1, 0, 1, 3), (1, 2), 5),
              synth.ConvShape("gb2", 1, 160, 33, 45, 40, 3, 3, (2, 1), (1, 1, 1, 1), (1, 1), 20)):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        _check(orc, s, x, w, rng, tag="grouped")


@pytest.mark.parametrize("batch", [1, 8])
def test_squeeze_excitation(orc, batch):
    """1x1 convolutions of 1x1 planes (single-column products at batch 1)."""
    rng = np.random.default_rng(980 + batch)
    shapes = synth.mobilenetv3_large_se(batch)
    for s in (shapes[0], shapes[1], shapes[-2], shapes[-1]):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)))
        _check(orc, s, x, w, rng, tag=f"se b{batch}")


def test_no_epilogue_through_the_epilogue_entry(orc):
    """og_conv2d_f32_epi with no bias, no activation and no residual gives
    og_conv2d_f32_ex's bits."""
    t = torch()
    rng = np.random.default_rng(990)
    s = synth.ConvShape("plain", 2, 16, 13, 17, 24, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1)
    x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
    x = _specials(x, rng, 0.01)
    dx, dw = t.from_numpy(x).cuda(), t.from_numpy(w).cuda()
    for mode in MODES:
        y = t.empty(_out_shape(s), dtype=t.float32, device="cuda")
        og.set_stream(t.cuda.current_stream().cuda_stream)
        rc = og.lib().og_conv2d_f32_epi(s.N, s.Cin, s.H, s.W, s.Cout, 1, 3, 3, 1, 1, 1, 1, 1, 1,
                                        1, 1, dx.data_ptr(), dw.data_ptr(), None, og.ACT_NONE,
                                        None, y.data_ptr(), mode)
        assert rc == og.OG_OK
        want = orc.conv2d(x, w, mode, stride=s.stride, pad=s.pad, dil=s.dil)
        assert_same_bits(to_host(y), want, f"plain epi mode {mode}")
