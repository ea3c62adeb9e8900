"""The hand-worked cases and the arithmetic discriminators, run through every
kernel variant on the GPU and compared bit for bit with the oracle and with
values fixed by the pages or by first principles ("Exact mode", section
"Checking it": NaN, infinity, signed-zero and subnormal inputs through every
path).

Each hand case of ``tests/golden/hand_cases.jsonl`` is planted in a product
large enough to span several tiles of every variant: the case's row of A
holds its terms at increasing positions of k and zeros elsewhere (a zero
term adds a signed zero, which leaves the sum unchanged: the sum is never
-0), its column of B holds the case's other operands there; the rest is
random.  The planted output must equal the case's stored bits, and every
output the oracle's.

Discriminators:
  * the sign of an underflowing fused sum: products far below the smallest
    subnormal, negative in odd columns, with k running past the last whole
    chunk of every kernel; fast mode gives -0 there and exact mode +0, so a
    k tail padded with terms that add +0 (turning -0 into +0) would show;
  * fused against unfused: output (i, j) sums c + a*b with c = -round(a*b)
    placed before a*b.  Separately rounded, the sum is +0; fused, it is the
    rounding error of a*b, computed here exactly in float64;
  * subnormal products and sums: operands near 2^-70, so every product and
    partial sum is subnormal (flush-to-zero anywhere would show);
  * order: terms of mixed magnitude (2^24 beside ones) whose sum depends on
    the order they are added in, products and convolutions (each output's
    taps in (channel, kernel row, kernel column) order).
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import oracle
import pins
import synth
from gpu_util import assert_same_bits, bits, say, to_device_strided, to_host, torch

pytestmark = pytest.mark.gpu
MODES = {"exact": og.EXACT, "fast": og.FAST}
VARIANTS = list(range(0, 21)) + [26, 27, 28, 29, 30, 31, 32, 33]  # tiles, then the halo and panel kernels
M, N, K = 300, 520, 40  # several tiles of the largest tile shapes, each ending inside


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def auto_variant():
    og.set_variant(0)
    yield
    og.set_variant(0)


def _gpu_gemm(A, B, mode, ldc_pad=1):
    m, k = A.shape
    n = B.shape[1]
    dA, _ = to_device_strided(A, max(1, k) + 1, 1)
    dB, _ = to_device_strided(B, max(1, n) + 3, 2)
    fill = np.full((m, n), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
    dC, _ = to_device_strided(fill, n + ldc_pad, 0, gap_bits=synth.GAP_OUT_BITS)
    og.gemm(dA, dB, mode, out=dC)
    torch().cuda.synchronize()
    return to_host(dC)


def _gpu_conv(x, w, s, mode):
    t = torch()
    y = og.conv2d(t.from_numpy(x).cuda(), t.from_numpy(w).cuda(), stride=s.stride, pad=s.pad,
                  dil=s.dil, groups=s.groups, mode=mode)
    return to_host(y)


def _planted_gemm(rng, mname):
    """A random M x N x K product with the hand cases of this mode planted at
    distinct rows and columns; returns A, B and {(i, j): expected bits}."""
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    want = {}
    cases = [c for c in pins.load_hand_cases()
             if c["op"] == "gemm" and c["k"] > 0 and mname in c["modes"]]
    for t, c in enumerate(cases):
        i, j = 17 + 29 * t, 5 + 51 * t
        assert i < M and j < N
        pos = np.sort(rng.choice(K, size=c["k"], replace=False))
        A[i, :] = 0.0
        A[i, pos] = pins.from_hex(c["A"], (c["k"],))
        B[pos, j] = pins.from_hex(c["B"], (c["k"],))
        want[(i, j)] = int(c["C"][0], 16)
    return A, B, want


@pytest.mark.parametrize("variant", VARIANTS)
def test_hand_cases_planted_in_every_variant(orc, variant):
    """W1-W6 (order, overflow, fused/unfused, -0, NaN, subnormals) inside a
    product of several tiles, and W7 (k = 0), on each variant."""
    rng = np.random.default_rng(900 + variant)
    og.set_variant(variant)
    for mname, mode in MODES.items():
        A, B, want = _planted_gemm(rng, mname)
        say(f"golden gemm variant {variant} mode {mname}")
        got = _gpu_gemm(A, B, mode)
        assert_same_bits(got, orc.gemm(A, B, mode), f"planted cases variant {variant} {mname}")
        u = bits(got)
        for (i, j), w in want.items():
            assert u[i, j] == w, f"hand case at ({i}, {j}) variant {variant} {mname}: " \
                                 f"{u[i, j]:08x} != {w:08x}"
        # W7: k = 0 stores +0 everywhere
        got0 = _gpu_gemm(np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32), mode)
        assert np.all(bits(got0) == 0), f"k = 0 variant {variant} {mname}"


@pytest.mark.parametrize("variant", VARIANTS)
def test_underflow_to_minus_zero(orc, variant):
    """Fast mode keeps the -0 of an underflowing fused sum through the padding
    of k's last chunk, for k below, at and past each kernel's chunk sizes."""
    rng = np.random.default_rng(930 + variant)
    og.set_variant(variant)
    for m, n, k in ((300, 520, 40), (37, 130, 1), (70, 64, 16), (70, 64, 64), (9, 200, 129),
                    (5, 300, 300), (1, 4096, 300), (130, 66, 145)):
        A, B, fast = pins.underflow_family(rng, m, n, k)
        for mname, mode in MODES.items():
            say(f"underflow sign variant {variant} {m}x{n}x{k} mode {mname}")
            got = _gpu_gemm(A, B, mode)
            want = fast if mode == og.FAST else np.zeros((m, n), np.uint32)
            assert_same_bits(got, want.view(np.float32), f"underflow {m}x{n}x{k} v{variant} {mname}")
    # convolutions: channels past a chunk, and padding taps (+0 inputs times
    # negative weights add -0, which keeps -0)
    for s in CONV_SHAPES + [synth.ConvShape("u3x3", 1, 37, 6, 7, 20, 3, 3, (1, 1), (1, 1, 1, 1)),
                            # weight rows of whole quads: the halo kernel's shapes
                            synth.ConvShape("u3x3q", 2, 36, 6, 7, 20, 3, 3, (1, 1), (1, 1, 1, 1)),
                            synth.ConvShape("u3x3s2", 1, 20, 9, 8, 12, 3, 3, (2, 2), (1, 1, 1, 1)),
                            synth.ConvShape("u1x1", 2, 130, 5, 6, 9, 1, 1)]:
        x = np.full((s.N, s.Cin, s.H, s.W), 2.0 ** -100, np.float32)
        w = (-rng.uniform(1, 2, (s.Cout, s.Cin // s.groups, s.KH, s.KW)) * 2.0 ** -60).astype(
            np.float32)
        for mname, mode in MODES.items():
            say(f"underflow sign conv variant {variant} {s} mode {mname}")
            got = _gpu_conv(x, w, s, mode)
            want = orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)
            assert np.all(bits(want) == (0x80000000 if mode == og.FAST else 0))
            assert_same_bits(got, want, f"underflow conv {s.name} v{variant} {mname}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_fused_against_unfused(orc, variant):
    """Exact mode gives +0 everywhere (the product rounded before it meets
    -round(a*b)); fast mode gives the rounding error of each product (one
    fused multiply-add): the matrix-core, VALU, DPP and lane paths alike."""
    rng = np.random.default_rng(950 + variant)
    og.set_variant(variant)
    A, B, fused = pins.fused_unfused_family(rng)
    assert np.count_nonzero(fused) > 0.9 * fused.size
    for mname, mode in MODES.items():
        say(f"fused/unfused variant {variant} mode {mname}")
        got = _gpu_gemm(A, B, mode)
        assert_same_bits(got, orc.gemm(A, B, mode), f"discriminator variant {variant} {mname}")
        want = np.zeros_like(fused) if mode == og.EXACT else fused
        assert_same_bits(got, want, f"discriminator from first principles {variant} {mname}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_subnormal_products_and_sums(orc, variant):
    """Operands near 2^-70 (products near 2^-140, below the normal range):
    every product and sum is subnormal; both modes keep them."""
    rng = np.random.default_rng(970 + variant)
    og.set_variant(variant)
    A = (rng.standard_normal((M, K)) * 2.0 ** -70).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 2.0 ** -70).astype(np.float32)
    for mname, mode in MODES.items():
        say(f"subnormal products variant {variant} mode {mname}")
        got = _gpu_gemm(A, B, mode)
        want = orc.gemm(A, B, mode)
        assert np.count_nonzero(bits(want) & 0x7FFFFFFF) > 0.9 * want.size
        assert_same_bits(got, want, f"subnormal variant {variant} {mname}")


def _absorbing(rng, shape):
    """Magnitudes 2^24 and 2^23 among ones and halves: sums that depend on
    the order of their terms."""
    v = rng.choice(np.array([2.0 ** 24, 2.0 ** 23, 1.0, 1.0, 1.0, 0.5, 0.5, 3.0]), size=shape)
    return (v * rng.choice([-1.0, 1.0], size=shape)).astype(np.float32)


@pytest.mark.parametrize("variant", VARIANTS)
def test_order_sensitive_product(orc, variant):
    rng = np.random.default_rng(990 + variant)
    og.set_variant(variant)
    A = _absorbing(rng, (M, K))
    B = rng.choice(np.array([1.0, 1.0, 0.5, -1.0], np.float32), size=(K, N)).astype(np.float32)
    for mname, mode in MODES.items():
        say(f"order-sensitive product variant {variant} mode {mname}")
        assert_same_bits(_gpu_gemm(A, B, mode), orc.gemm(A, B, mode),
                         f"order-sensitive product variant {variant} {mname}")


CONV_SHAPES = [
    # a regular 3x3 with padding and stride, two groups (the chain, lane and tile paths)
    synth.ConvShape("o3x3", 2, 12, 11, 10, 40, 3, 3, (1, 2), (1, 1, 1, 0), (1, 1), 2),
    # 1x1 planes read in place, and strided
    synth.ConvShape("o1x1", 2, 20, 7, 9, 70, 1, 1),
    synth.ConvShape("o1x1s2", 2, 20, 7, 9, 70, 1, 1, (2, 2)),
    # W9's window: 2 channels per group, 2x2
    synth.ConvShape("o2x2", 2, 4, 10, 10, 40, 2, 2, (1, 1), (0, 0, 0, 0), (1, 1), 2),
    # depthwise 3x3 and a grouped 3x3 with few output channels per group
    synth.ConvShape("odw", 2, 16, 12, 12, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 16),
    synth.ConvShape("ogr", 2, 32, 12, 12, 32, 3, 3, (2, 2), (2, 2, 2, 2), (2, 2), 4),
]


@pytest.mark.parametrize("variant", VARIANTS)
def test_convolution_cases_in_every_variant(orc, variant):
    """Convolutions on every variant: order-sensitive taps (x = 1 inside the
    plane, weights of mixed magnitude), W8 (an infinite weight on a padding
    tap gives NaN) and W9 ((c, ky, kx) order gives exactly 2)."""
    rng = np.random.default_rng(1010 + variant)
    og.set_variant(variant)
    w9 = [c for c in pins.load_hand_cases() if c["id"] == "W9"][0]
    for s in CONV_SHAPES:
        x = np.ones((s.N, s.Cin, s.H, s.W), np.float32)
        w = _absorbing(rng, (s.Cout, s.Cin // s.groups, s.KH, s.KW))
        planted_nan = None
        if s.name == "o2x2":
            # W9 on output channel 0 (group 0): every output of that channel is 2
            w[0] = pins.from_hex(w9["w"], (2, 2, 2))
        elif s.pad[0] >= 1 and s.pad[1] >= 1:
            # W8: output channel 1, its group's first channel, tap (0, 0) infinite: the
            # outputs of the first row and column take that tap from the padding
            w[1, 0, 0, 0] = np.inf
            planted_nan = 1
        for mname, mode in MODES.items():
            say(f"golden conv variant {variant} {s} mode {mname}")
            got = _gpu_conv(x, w, s, mode)
            want = orc.conv2d(x, w, mode, groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)
            assert_same_bits(got, want, f"golden conv variant {variant} {s.name} {mname}")
            if s.name == "o2x2":
                assert np.all(bits(got[:, 0]) == 0x40000000), f"W9 variant {variant} {mname}"
            if planted_nan is not None:
                u = bits(got[:, planted_nan])
                assert np.all(u[:, 0, :] == 0x7FC00000) and np.all(u[:, :, 0] == 0x7FC00000), \
                    f"W8 variant {variant} {s.name} {mname}"
