"""GPU parity of the implicit-GEMM convolution: libog (through its C ABI)
against the CPU oracle's direct convolution, bit for bit, exact and fast.

Cases: small random shapes covering stride, asymmetric padding, dilation,
groups (depthwise included) and batch, with special values; and every output
of the full-size workloads: the 53 layers of ResNet-50 v1.5 at batch 1 and 8,
the grouped dilated strided convolution and the 1-D convolution (H = 1), the
SHA-256 of the GPU's outputs, the oracle's and the stored ones printed at the
end of the session and equal.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import full_size
import oracle
import synth
from gpu_util import assert_same_bits, record_hashes, say, sha256, to_host, torch

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


def _gpu_conv(x, w, s: synth.ConvShape, mode):
    t = torch()
    dx = t.from_numpy(x).cuda()
    dw = t.from_numpy(w).cuda()
    y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups, mode=mode)
    return to_host(y)


def _oracle(orc, x, w, s, mode):
    return orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)


def _random_shapes(rng, count):
    shapes = []
    while len(shapes) < count:
        G = int(rng.choice([1, 1, 2, 3, 4]))
        cin_g = int(rng.integers(1, 9))
        cout_g = int(rng.integers(1, 40))
        KH, KW = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        H, W = int(rng.integers(1, 23)), int(rng.integers(1, 23))
        st = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dl = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        pad = tuple(int(p) for p in rng.integers(0, 4, size=4))
        if H + pad[0] + pad[2] - dl[0] * (KH - 1) - 1 < 0:
            continue
        if W + pad[1] + pad[3] - dl[1] * (KW - 1) - 1 < 0:
            continue
        shapes.append(synth.ConvShape(f"rand{len(shapes)}", int(rng.integers(1, 4)), G * cin_g,
                                      H, W, G * cout_g, KH, KW, st, pad, dl, G))
    return shapes


def _with_specials(a, rng, frac):
    a = a.copy()
    synth.inject_specials(a.reshape(a.shape[0], -1), frac, int(rng.integers(1 << 30)))
    return a


@pytest.mark.parametrize("mode", MODES)
def test_random_shapes(orc, mode):
    rng = np.random.default_rng(200 + mode)
    for s in _random_shapes(rng, 60):
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _with_specials(x, rng, 0.01)
        w = _with_specials(w, rng, 0.01)
        say(f"conv {s} mode {mode}")
        assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


@pytest.mark.parametrize("variant", list(range(1, 21)))
def test_variants_agree(orc, variant):
    rng = np.random.default_rng(300)
    og.set_variant(variant)
    shapes = [synth.ConvShape("v3x3", 2, 24, 13, 11, 40, 3, 3, (1, 2), (1, 0, 2, 1), (2, 1), 2),
              synth.ConvShape("v1x1", 3, 20, 9, 7, 70, 1, 1)]
    for s in shapes:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        for mode in MODES:
            say(f"conv variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"variant {variant} {s} mode {mode}")


@pytest.mark.parametrize("variant", [10, 11, 12, 13, 14, 15, 16])
def test_chain_kernel_shapes(orc, variant):
    """The chain kernel on 3x3 and 1x1 windows (strided, padded, dilated,
    grouped, several chunks of channels) and its fallback for other windows."""
    rng = np.random.default_rng(400 + variant)
    og.set_variant(variant)
    shapes = [synth.ConvShape("c3", 2, 40, 9, 11, 12, 3, 3, (2, 1), (1, 0, 2, 1), (2, 1)),
              synth.ConvShape("c3g", 1, 34, 7, 7, 10, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 2),
              synth.ConvShape("c1s", 2, 70, 9, 8, 9, 1, 1, (2, 2)),
              synth.ConvShape("c1p", 3, 130, 5, 6, 5, 1, 1),
              synth.ConvShape("c5", 1, 6, 9, 9, 7, 5, 3, (1, 2), (2, 1, 2, 1)),
              # 3x3 row loads: stride 2, the narrowest row, pads 0 and 1 on either side
              synth.ConvShape("c3s2", 1, 20, 9, 8, 11, 3, 3, (2, 2), (1, 1, 1, 1)),
              synth.ConvShape("c3w3", 2, 9, 5, 3, 6, 3, 3, (1, 1), (1, 1, 1, 1)),
              synth.ConvShape("c3p01", 1, 18, 6, 10, 5, 3, 3, (1, 3), (0, 0, 1, 1)),
              # pads of 2: the tap loads
              synth.ConvShape("c3p2", 1, 10, 6, 7, 5, 3, 3, (1, 1), (2, 2, 2, 2))]
    for s in shapes:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _with_specials(x, rng, 0.01)
        w = _with_specials(w, rng, 0.01)
        for mode in MODES:
            say(f"conv chain variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"chain {variant} {s} mode {mode}")


HALO_SHAPES = [
    # rows past Cout, channels in three chunks (the last one short)
    synth.ConvShape("h14", 2, 40, 14, 14, 36, 3, 3, (1, 1), (1, 1, 1, 1)),
    # rows 16 bytes wide: 16-byte halo loads
    synth.ConvShape("h28", 1, 20, 28, 28, 24, 3, 3, (1, 1), (1, 1, 1, 1)),
    synth.ConvShape("h56s2", 2, 16, 56, 56, 8, 3, 3, (2, 2), (1, 1, 1, 1)),
    # wide rows: halos of two buffers (two barriers per chunk)
    synth.ConvShape("h56", 1, 36, 56, 56, 20, 3, 3, (1, 1), (1, 1, 1, 1)),
    # 49 pixels per image, three images
    synth.ConvShape("h7", 3, 36, 7, 7, 70, 3, 3, (1, 1), (1, 1, 1, 1)),
    # groups, dilation, strides on one axis, asymmetric padding
    synth.ConvShape("hg", 2, 40, 13, 11, 40, 3, 3, (1, 2), (1, 0, 2, 1), (2, 1), 2),
    # narrow images: a tile of 64 pixels spans many rows
    synth.ConvShape("hw3", 1, 20, 70, 3, 12, 3, 3, (1, 1), (1, 1, 1, 1)),
    synth.ConvShape("hw1", 1, 12, 100, 1, 5, 3, 3, (1, 1), (1, 1, 1, 1)),
    # pads of 2, four channels
    synth.ConvShape("hp2", 2, 4, 9, 10, 19, 3, 3, (1, 1), (2, 2, 2, 2)),
    # a halo too wide to stage, horizontal dilation 2, weight rows not of
    # whole quads (Cin/G = 9) and a 1x1 window: the automatic choice runs
    synth.ConvShape("hwide", 1, 8, 9, 300, 6, 3, 3, (1, 1), (1, 1, 1, 1)),
    synth.ConvShape("hdw2", 1, 16, 9, 12, 20, 3, 3, (1, 1), (1, 2, 1, 2), (1, 2)),
    synth.ConvShape("hodd", 1, 9, 12, 10, 7, 3, 3, (1, 1), (1, 1, 1, 1)),
    synth.ConvShape("h1x1", 2, 20, 9, 7, 30, 1, 1),
]


@pytest.mark.parametrize("variant", [26, 27, 28, 31, 32, 33])
def test_halo_kernel_shapes(orc, variant):
    """The halo kernel (3x3 windows; on the matrix cores, exact mode's
    products there and its sums on the VALU, fast mode's chains there; or
    in DPP steps on the VALU) bit for bit against the oracle; on shapes it
    does not take the variant runs the automatic choice."""
    rng = np.random.default_rng(500 + variant)
    og.set_variant(variant)
    for s in HALO_SHAPES:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _with_specials(x, rng, 0.01)
        w = _with_specials(w, rng, 0.01)
        for mode in MODES:
            say(f"conv halo variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"halo {variant} {s} mode {mode}")


PANEL_SHAPES = [
    # 1x1 read in place, 16-byte rows (64 pixels) and not (49), channels
    # ending inside a 32-step chunk, rows past Cout
    synth.ConvShape("p8", 2, 40, 8, 8, 36, 1, 1),
    synth.ConvShape("p7", 3, 70, 7, 7, 20, 1, 1),
    synth.ConvShape("p3", 1, 3, 9, 12, 5, 1, 1),
    # strided and padded 1x1: the gathered form
    synth.ConvShape("p14s2", 2, 64, 14, 14, 33, 1, 1, (2, 2)),
    synth.ConvShape("ppad", 2, 20, 6, 9, 17, 1, 1, (1, 2), (1, 0, 2, 1)),
    # groups
    synth.ConvShape("pg", 2, 64, 10, 10, 48, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 4),
    # a 3x3 window: the automatic choice runs
    synth.ConvShape("p3x3", 1, 16, 9, 9, 8, 3, 3, (1, 1), (1, 1, 1, 1)),
]


@pytest.mark.parametrize("variant", [29, 30])
def test_panel_kernel_shapes(orc, variant):
    """The panel kernel (fast mode, 1x1 windows) bit for bit against the
    oracle; in exact mode, and on other windows, the automatic choice."""
    rng = np.random.default_rng(600 + variant)
    og.set_variant(variant)
    for s in PANEL_SHAPES:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _with_specials(x, rng, 0.01)
        w = _with_specials(w, rng, 0.01)
        for mode in MODES:
            say(f"conv panel variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"panel {variant} {s} mode {mode}")


GROUPED_SHAPES = [
    # the grouped, dilated, strided workload's own form, smaller
    synth.ConvShape("g8x8", 2, 64, 20, 18, 64, 3, 3, (2, 2), (2, 2, 2, 2), (2, 2), 8),
    # Cout/G of 1, 3, 5 (rows per lane rounded up), Cin/G from 2 to 20 (two channel blocks)
    synth.ConvShape("g1", 1, 8, 9, 70, 4, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 4),
    synth.ConvShape("g3", 3, 40, 11, 13, 6, 3, 3, (1, 2), (0, 1, 2, 0), (1, 1), 2),
    synth.ConvShape("g5", 1, 100, 17, 9, 25, 3, 3, (2, 1), (1, 0, 1, 3), (1, 2), 5),
    synth.ConvShape("g8w", 2, 32, 65, 3, 32, 3, 3, (1, 1), (1, 1, 1, 1), (3, 1), 4),
    # wider planes: stride 2 and dilation 2 across, dilation 2 down, strides
    # on one axis, two channel blocks (Cin/G = 20), asymmetric padding
    synth.ConvShape("gb1", 2, 48, 40, 50, 32, 3, 3, (1, 2), (2, 1, 2, 3), (2, 2), 8),
    synth.ConvShape("gb2", 1, 160, 33, 45, 40, 3, 3, (2, 1), (1, 1, 1, 1), (1, 1), 20),
    synth.ConvShape("gb3", 1, 80, 20, 30, 20, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 4),
]


@pytest.mark.parametrize("variant", [0, 3, 7, 19])
def test_grouped_direct_kernel(orc, variant):
    """Grouped 3x3 convolutions with few output channels per group run the
    grouped direct kernel (0 and 19) with the implicit product's bits (3, 7)."""
    og.set_variant(variant)
    rng = np.random.default_rng(450)
    for s in GROUPED_SHAPES:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = _with_specials(x, rng, 0.005)
        w = _with_specials(w, rng, 0.01)
        for mode in MODES:
            say(f"conv grouped variant {variant} {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode),
                             f"grouped variant {variant} {s} mode {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_mobilenetv3_large_all_convs(orc, mode):
    """The 46 convolutions of MobileNetV3-large at batch 1 (stem, 1x1
    expansions and projections, depthwise, last 1x1), every output."""
    for i, s in enumerate(synth.mobilenetv3_large_convs(1)):
        x, w = synth.conv_inputs(s, synth.seed_for(8, 500 + i))
        say(f"mobilenetv3 conv {s} mode {mode}")
        assert sha256(_gpu_conv(x, w, s, mode)) == sha256(_oracle(orc, x, w, s, mode)), f"{s}"


def test_whisper_frontend_convs(orc):
    """The Whisper-small encoder's two 1-D convolutions (as H = 1), every output."""
    for i, s in enumerate(synth.whisper_small_frontend()):
        x, w = synth.conv_inputs(s, synth.seed_for(8, 600 + i))
        for mode in MODES:
            say(f"whisper conv {s} mode {mode}")
            assert_same_bits(_gpu_conv(x, w, s, mode), _oracle(orc, x, w, s, mode), f"{s} mode {mode}")


def test_padding_tap_meets_infinite_weight(orc):
    """An infinite weight on a padding tap gives NaN (padding taps are real products)."""
    s = synth.ConvShape("w8", 1, 1, 1, 1, 1, 3, 3, (1, 1), (1, 1, 1, 1))
    x = np.array([[[[2.0]]]], np.float32)
    w = np.ones((1, 1, 3, 3), np.float32)
    w[0, 0, 0, 0] = np.inf
    for mode in MODES:
        y = _gpu_conv(x, w, s, mode)
        assert y.view(np.uint32).ravel()[0] == 0x7FC00000


def _full_conv(orc, name):
    """Every output of every layer of a full-size workload, both modes,
    against the oracle; the digests of GPU, oracle and stored values equal."""
    stored = full_size.stored()[name]
    dig = {m: (full_size.Digest(), full_size.Digest()) for m in full_size.MODES}
    for i, (s, x, w) in enumerate(full_size.conv_layers(name)):
        for mname, mode in full_size.MODES.items():
            say(f"{name} layer {i} {s} mode {mname}")
            got = _gpu_conv(x, w, s, mode)
            want = full_size.oracle_conv(orc, s, x, w, mode)
            assert_same_bits(got, want, f"{name} layer {i} {s.name} mode {mname}")
            dig[mname][0].add(got)
            dig[mname][1].add(want)
    for mname in full_size.MODES:
        dg, do = dig[mname][0].hex(), dig[mname][1].hex()
        record_hashes(name, mname, dg, do, stored[mname])
        assert dg == do == stored[mname], f"{name} {mname}: digests differ"


def test_resnet50_batch1_all_layers(orc):
    """All 53 layers of the chain at batch 1, every output, both modes."""
    _full_conv(orc, "resnet50_b1")


def test_resnet50_batch8_all_layers(orc):
    """All 53 layers of the chain at batch 8, every output, both modes."""
    _full_conv(orc, "resnet50_b8")


def test_grouped_dilated_full(orc):
    _full_conv(orc, "grouped_dilated")


def test_conv1d_h1_full(orc):
    """The 1-D convolution (8 x 512 -> 512 channels, 4096 wide, KW = 5, pads 2
    on the width only): every output; and image 0 alone (batch invariance)."""
    _full_conv(orc, "conv1d_h1")
    s, x, w = next(full_size.conv_layers("conv1d_h1"))
    for mode in MODES:
        say(f"conv1d image 0 mode {mode}")
        got = _gpu_conv(np.ascontiguousarray(x[:1]), w, s.with_batch(1), mode)
        assert_same_bits(got, full_size.oracle_conv(orc, s.with_batch(1), x[:1].copy(), w, mode),
                         f"conv1d image 0 mode {mode}")
