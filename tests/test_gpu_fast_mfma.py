"""GPU checks of mode 2 (fast under a stated tolerance): every result within
|c - r| <= 4e-6 * sqrt(K) * S + 1e-30 of the exact sum, with the exact
result's class where that is not finite (oracle/tolerance.py, pinned by
tests/test_tolerance_checker.py); NaN stored as 0x7FC00000; the same bits
from run to run.

Each split-k variant (21..25) is forced on products and convolutions whose
sizes end inside tiles and inside the 16-tap chunks of k, with row strides
and special values; the automatic choice runs every full-size workload: the
256^3 and 4096^3 products, the ragged one with its row strides, prefill and
skinny, the ResNet-50 chain at batch 1 and 8, the grouped dilated and the
1-D convolutions.  Bits are not compared with the oracle's (mode 2 has no
single correct bit pattern); the parity of mode 2 is its bound.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import full_size
import oracle
import synth
from gpu_util import bits, say, to_device_strided, to_host, torch
from oracle import tolerance

pytestmark = pytest.mark.gpu
SPLIT = [21, 22, 23, 24, 25]
M2 = og.FAST_MFMA


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def auto_variant():
    og.set_variant(0)
    yield
    og.set_variant(0)


def _mixed(rng, shape, frac):
    v = rng.standard_normal(shape).astype(np.float32)
    if frac > 0 and v.size:
        synth.inject_specials(v.reshape(shape[0], -1), frac, int(rng.integers(1 << 30)))
    return v


def _gemm(A, B, mode, lda, ldb, ldc, nt=False):
    m = A.shape[0]
    n = B.shape[0] if nt else B.shape[1]
    dA, _ = to_device_strided(A, lda)
    dB, _ = to_device_strided(B, ldb)
    fill = np.full((m, n), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
    dC, flatC = to_device_strided(fill, ldc, gap_bits=synth.GAP_OUT_BITS)
    (og.gemm_nt if nt else og.gemm)(dA, dB, mode, out=dC)
    torch().cuda.synchronize()
    return to_host(dC), to_host(flatC), (dA, dB, dC)


def _assert_within(rep, what):
    assert rep["ok"], f"{what}: {rep}"


def _assert_canonical_nan(got, what):
    u = bits(got)
    nan = np.isnan(got)
    assert np.all(u[nan] == 0x7FC00000), f"{what}: a NaN is not 0x7FC00000"


GEMM_SHAPES = [(1, 1, 1), (1, 70, 0), (17, 33, 1), (16, 16, 16), (19, 37, 17), (33, 65, 100),
               (1, 300, 531), (70, 5, 64), (130, 100, 1531), (5, 260, 4096)]


@pytest.mark.parametrize("variant", SPLIT)
def test_split_variant_products(orc, variant):
    rng = np.random.default_rng(1200 + variant)
    og.set_variant(variant)
    for (m, n, k) in GEMM_SHAPES:
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        lda, ldb, ldc = max(1, k) + int(rng.integers(0, 5)), max(1, n) + int(rng.integers(0, 5)), n + 3
        say(f"mode 2 variant {variant} gemm {m}x{n}x{k}")
        got, flatC, dev = _gemm(A, B, M2, lda, ldb, ldc)
        u = flatC.view(np.uint32).reshape(-1)
        idx = np.arange(m)[:, None] * ldc + np.arange(n)[None, :]
        mask = np.ones(u.shape, bool)
        mask[idx.ravel()] = False
        assert np.all(u[mask] == synth.GAP_OUT_BITS), "an element outside C was written"
        _assert_within(tolerance.check_gemm(A, B, got, orc.gemm(A, B, 0)),
                       f"variant {variant} {m}x{n}x{k}")
        _assert_canonical_nan(got, f"variant {variant} {m}x{n}x{k}")
        if k == 0:
            assert np.all(bits(got) == 0)
        # the same bits again
        og.gemm(dev[0], dev[1], M2, out=dev[2])
        assert np.array_equal(bits(to_host(dev[2])), bits(got)), "a second run differs"


@pytest.mark.parametrize("variant", SPLIT)
def test_split_variant_products_nt(orc, variant):
    """The product with B given as n x k, 16-byte rows and not."""
    rng = np.random.default_rng(1300 + variant)
    og.set_variant(variant)
    for (m, n, k, ldb) in ((1, 300, 512, 512), (19, 37, 17, 19), (33, 65, 100, 100),
                           (70, 130, 516, 520)):
        A = _mixed(rng, (m, k), 0.01)
        Bt = _mixed(rng, (n, k), 0.01)
        say(f"mode 2 variant {variant} gemm_nt {m}x{n}x{k}")
        got, _, _ = _gemm(A, Bt, M2, k, ldb, n, nt=True)
        Bc = np.ascontiguousarray(Bt.T)
        _assert_within(tolerance.check_gemm(A, Bc, got, orc.gemm(A, Bc, 0)),
                       f"nt variant {variant} {m}x{n}x{k}")


CONV_SHAPES = [
    synth.ConvShape("s3x3", 2, 24, 13, 11, 40, 3, 3, (1, 2), (1, 0, 2, 1), (2, 1), 2),
    synth.ConvShape("s1x1", 3, 20, 9, 7, 70, 1, 1),
    synth.ConvShape("s1x1s2", 2, 64, 14, 14, 36, 1, 1, (2, 2)),
    synth.ConvShape("s7x7", 1, 3, 40, 40, 16, 7, 7, (2, 2), (3, 3, 3, 3)),
    synth.ConvShape("s5x3", 2, 6, 9, 9, 7, 5, 3, (1, 2), (2, 1, 2, 1)),
    synth.ConvShape("sdw", 2, 16, 12, 12, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 16),
    synth.ConvShape("sgr", 2, 64, 20, 18, 64, 3, 3, (2, 2), (2, 2, 2, 2), (2, 2), 8),
    synth.ConvShape("s1d", 2, 40, 1, 300, 24, 1, 5, (1, 1), (0, 2, 0, 2)),
    synth.ConvShape("sdeep", 1, 512, 7, 7, 48, 3, 3, (1, 1), (1, 1, 1, 1)),
]


def _conv(x, w, s, mode, **epi):
    t = torch()
    y = og.conv2d(t.from_numpy(x).cuda(), t.from_numpy(w).cuda(), stride=s.stride, pad=s.pad,
                  dil=s.dil, groups=s.groups, mode=mode, **epi)
    return to_host(y)


def _conv_check(orc, x, w, s, got, what):
    kw = dict(groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)
    exact = orc.conv2d(x, w, 0, **kw)
    _assert_within(tolerance.check_conv(x, w, got, exact, **kw), what)
    _assert_canonical_nan(got, what)


@pytest.mark.parametrize("variant", SPLIT)
def test_split_variant_convolutions(orc, variant):
    rng = np.random.default_rng(1400 + variant)
    og.set_variant(variant)
    for s in CONV_SHAPES:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        x = x.copy()
        synth.inject_specials(x.reshape(x.shape[0], -1), 0.002, int(rng.integers(1 << 30)))
        say(f"mode 2 variant {variant} conv {s}")
        got = _conv(x, w, s, M2)
        _conv_check(orc, x, w, s, got, f"variant {variant} {s.name}")
        assert np.array_equal(bits(_conv(x, w, s, M2)), bits(got)), "a second run differs"


@pytest.mark.parametrize("variant", [0, 21, 23])
def test_epilogue_follows_the_sum(orc, variant):
    """With the epilogue, mode 2 stores bias, ReLU and residual applied to the
    same sum it stores without one (the oracle's epilogue on the plain result,
    bit for bit)."""
    rng = np.random.default_rng(1500 + variant)
    og.set_variant(variant)
    for s in CONV_SHAPES[:3] + CONV_SHAPES[-1:]:
        x, w = synth.conv_inputs(s, int(rng.integers(1 << 30)), "uniform")
        say(f"mode 2 epilogue variant {variant} {s}")
        plain = _conv(x, w, s, M2)
        b = rng.standard_normal(s.Cout).astype(np.float32)
        r = rng.standard_normal(plain.shape).astype(np.float32)
        t = torch()
        fused = _conv(x, w, s, M2, bias=t.from_numpy(b).cuda(), act="relu",
                      residual=t.from_numpy(r).cuda())
        want = orc.conv_epilogue(plain, b, 1, r)
        assert np.array_equal(bits(fused), bits(want)), f"epilogue variant {variant} {s.name}"


@pytest.mark.parametrize("variant", [1, 3, 10, 17, 20])
def test_forced_fast_variant_runs_fast_mode(orc, variant):
    """In mode 2 a forced variant 1..20 runs that fast-mode kernel: the bits of
    fast mode."""
    rng = np.random.default_rng(1600 + variant)
    og.set_variant(variant)
    A = rng.standard_normal((131, 97)).astype(np.float32)
    B = rng.standard_normal((97, 301)).astype(np.float32)
    say(f"mode 2 forced fast variant {variant}")
    got, _, _ = _gemm(A, B, M2, 97, 301, 301)
    assert np.array_equal(bits(got), bits(orc.gemm(A, B, 1)))


# ---------------------------------------------------------------------------
# the full-size workloads, the automatic choice
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(full_size.GEMMS))
def test_full_size_products(orc, name):
    c = full_size.gemm_case(name)
    say(f"mode 2 {name}")
    got, _, dev = _gemm(c.A, c.B, M2, c.lda, c.ldb, c.ldc)
    say(f"oracle exact {name}")
    exact = full_size.oracle_gemm(orc, c, 0)
    rep = tolerance.check_gemm(c.A, c.B, got, exact)
    say(f"mode 2 {name}: {rep}")
    _assert_within(rep, name)
    _assert_canonical_nan(got, name)
    og.gemm(dev[0], dev[1], M2, out=dev[2])
    assert np.array_equal(bits(to_host(dev[2])), bits(got)), "a second run differs"


@pytest.mark.parametrize("name", list(full_size.CONVS))
def test_full_size_convolutions(orc, name):
    worst = 0.0
    for i, (s, x, w) in enumerate(full_size.conv_layers(name)):
        say(f"mode 2 {name} layer {i} {s}")
        got = _conv(x, w, s, M2)
        exact = full_size.oracle_conv(orc, s, x, w, 0)
        kw = dict(groups=s.groups, stride=s.stride, pad=s.pad, dil=s.dil)
        rep = tolerance.check_conv(x, w, got, exact, **kw)
        _assert_within(rep, f"{name} layer {i} {s.name}")
        worst = max(worst, rep["worst_ratio"])
    say(f"mode 2 {name}: worst error / bound {worst:.3g}")
