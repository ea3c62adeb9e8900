"""GPU parity of the product with a transposed right operand (og_gemm_nt_f32,
B given as n x k) and of the single-column products (n = 1 matrix products,
m = 1 transposed products, 1x1 convolutions of a 1x1 input at batch 1),
against the CPU oracle, bit for bit, exact and fast.

The oracle computes C = A * B with B = the transpose of the n x k operand
(a numpy transpose of the same values): each output is the same sum of the
same products in the same order ("Exact mode", section "Matrix product").
Cases: sizes 0..70 with random row strides, pointer offsets and special
values; every variant with a form for the transposed operand; the prefill
shape 512 x 4096 against 11008 x 4096 weights on sampled outputs and whole
rows; single rows and single columns up to 4096 x 4096 in full, aligned and
unaligned; the 16 squeeze-and-excitation convolutions of MobileNetV3-large
at batch 1 and 8, and a grouped one.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import oracle
import synth
from gpu_util import assert_same_bits, bits, say, to_device_strided, to_host, torch

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


def _mixed(rng, shape, special_frac, std=1.0):
    v = (std * rng.standard_normal(shape)).astype(np.float32)
    if special_frac > 0 and v.size:
        synth.inject_specials(v.reshape(shape[0], -1), special_frac, int(rng.integers(1 << 30)))
    return v


def _check_gaps(flatC, m, n, ldc, off):
    u = flatC.view(np.uint32)
    mask = np.ones(u.shape, bool)
    if m and n:
        idx = off + np.arange(m)[:, None] * ldc + np.arange(n)[None, :]
        mask[idx.ravel()] = False
    assert np.all(u[mask] == synth.GAP_OUT_BITS), "an element outside C was written"


def _nt_gpu(A, Bt, mode, lda, ldb, ldc, offs=(0, 0, 0)):
    m, n = A.shape[0], Bt.shape[0]
    dA, _ = to_device_strided(A, lda, offs[0])
    dB, _ = to_device_strided(Bt, ldb, offs[1])
    fill = np.full((m, n), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
    dC, flatC = to_device_strided(fill, ldc, offs[2], gap_bits=synth.GAP_OUT_BITS)
    og.gemm_nt(dA, dB, mode, out=dC)
    torch().cuda.synchronize()
    return to_host(dC), to_host(flatC)


def _nt_oracle(orc, A, Bt, mode, rowwise=False):
    return orc.gemm(A, np.ascontiguousarray(Bt.T), mode, rowwise=rowwise)


SWEEP = [(d, 37, 45) for d in range(71)] + [(19, d, 45) for d in range(71)] + \
        [(19, 37, d) for d in range(71)]


@pytest.mark.parametrize("mode", MODES)
def test_nt_size_sweep_0_to_70(orc, mode):
    """Every size 0..70 in each dimension, random strides, offsets and special values."""
    rng = np.random.default_rng(800 + mode)
    say(f"gemm_nt sweep mode {mode}")
    for (m, n, k) in SWEEP:
        A = _mixed(rng, (m, k), 0.02)
        Bt = _mixed(rng, (n, k), 0.02)
        lda = max(1, k) + int(rng.integers(0, 5))
        ldb = max(1, k) + int(rng.integers(0, 5))
        ldc = max(1, n) + int(rng.integers(0, 5))
        offs = tuple(int(o) for o in rng.integers(0, 7, size=3))
        got, flatC = _nt_gpu(A, Bt, mode, lda, ldb, ldc, offs)
        assert_same_bits(got, _nt_oracle(orc, A, Bt, mode), f"nt {m}x{n}x{k} mode {mode}")
        _check_gaps(flatC, m, n, ldc, offs[2])


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5, 9, 17, 20])
def test_nt_variants_agree(orc, variant):
    """Every tile with a transposed-B form, aligned (16-byte loads) and not;
    a variant without one (9) runs as the automatic choice."""
    og.set_variant(variant)
    rng = np.random.default_rng(850)
    for (m, n, k, lda, ldb) in ((300, 517, 200, 200, 204), (70, 130, 61, 61, 67),
                                (257, 260, 516, 520, 516)):
        A = _mixed(rng, (m, k), 0.01)
        Bt = _mixed(rng, (n, k), 0.01)
        for mode in MODES:
            say(f"gemm_nt variant {variant} {m}x{n}x{k} mode {mode}")
            got, _ = _nt_gpu(A, Bt, mode, lda, ldb, n + 3)
            assert_same_bits(got, _nt_oracle(orc, A, Bt, mode),
                             f"nt variant {variant} {m}x{n}x{k} mode {mode}")


def test_nt_prefill_full(orc):
    """512 tokens x 4096 against 11008 x 4096 weights: every output (the
    oracle multiplies by the transpose of the weights, which it only moves)."""
    A = synth.normal((512, 4096), synth.seed_for(3, 20))
    Bt = synth.normal((11008, 4096), synth.seed_for(3, 21), 0.02)
    Bc = np.ascontiguousarray(Bt.T)
    dA, dB = torch().from_numpy(A).cuda(), torch().from_numpy(Bt).cuda()
    for mode in MODES:
        say(f"gemm_nt prefill mode {mode}")
        got = to_host(og.gemm_nt(dA, dB, mode))
        assert_same_bits(got, orc.gemm(A, Bc, mode, rowwise=True), f"nt prefill mode {mode}")


@pytest.mark.parametrize("model", ["bert_base_4096", "minilm_l6_4096", "whisper_small_enc_1500"])
def test_transformer_linear_layers_sampled(orc, model):
    """The linear layers of the transformer model rows (weights N x K):
    sampled outputs, corners and one whole row per shape."""
    rng = np.random.default_rng(900)
    for i, (name, m, n, k, _) in enumerate(synth.transformer_linear_shapes(model)):
        A = synth.normal((m, k), synth.seed_for(8, 10 * i))
        W = synth.normal((n, k), synth.seed_for(8, 10 * i + 1), 0.02)
        Wc = np.ascontiguousarray(W.T)
        dA, dW = torch().from_numpy(A).cuda(), torch().from_numpy(W).cuda()
        for mode in MODES:
            say(f"{model} {name} {m}x{n}x{k} mode {mode}")
            got = to_host(og.gemm_nt(dA, dW, mode))
            rows = np.concatenate([rng.integers(0, m, 1000), [0, 0, m - 1, m - 1]])
            cols = np.concatenate([rng.integers(0, n, 1000), [0, n - 1, 0, n - 1]])
            assert_same_bits(got[rows, cols], orc.gemm_at(A, Wc, rows, cols, mode),
                             f"{model} {name} sampled mode {mode}")
            r = int(rng.integers(0, m))
            assert_same_bits(got[r:r + 1], orc.gemm(A[r:r + 1], Wc, mode, rowwise=True),
                             f"{model} {name} row {r} mode {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_single_row_nt(orc, mode):
    """m = 1: one row against the rows of an n x k matrix, every output."""
    rng = np.random.default_rng(870 + mode)
    for (n, k, lda, ldb) in ((1, 1, 1, 1), (63, 17, 17, 17), (65, 64, 64, 64), (200, 300, 300, 303),
                             (129, 1000, 1000, 1000), (4096, 4096, 4096, 4096)):
        A = _mixed(rng, (1, k), 0.01)
        Bt = _mixed(rng, (n, k), 0.001, 0.02)
        say(f"gemm_nt single row n {n} k {k} ldb {ldb} mode {mode}")
        got, flatC = _nt_gpu(A, Bt, mode, lda, ldb, n + 2, (0, 1, 3))
        assert_same_bits(got, _nt_oracle(orc, A, Bt, mode), f"nt 1x{n}x{k} mode {mode}")
        _check_gaps(flatC, 1, n, n + 2, 3)


@pytest.mark.parametrize("mode", MODES)
def test_single_row_nt_streamed(orc, mode):
    """m = 1 with 16-byte aligned rows (k a multiple of 4): the row streamed
    against the N x K operand through the chain kernel; ragged n, k across
    chunk boundaries, padded row strides, every output."""
    rng = np.random.default_rng(875 + mode)
    for (n, k, ldb) in ((1, 4, 4), (15, 516, 520), (16, 128, 128), (17, 132, 136),
                        (300, 1000, 1004), (1000, 4096, 4096), (4096, 4096, 4096)):
        A = _mixed(rng, (1, k), 0.01)
        Bt = _mixed(rng, (n, k), 0.001, 0.02)
        say(f"gemm_nt single row (aligned) n {n} k {k} ldb {ldb} mode {mode}")
        got, flatC = _nt_gpu(A, Bt, mode, k, ldb, n + 2, (0, 0, 3))
        assert_same_bits(got, _nt_oracle(orc, A, Bt, mode), f"nt aligned 1x{n}x{k} mode {mode}")
        _check_gaps(flatC, 1, n, n + 2, 3)


@pytest.mark.parametrize("mode", MODES)
def test_few_rows_nt_streamed(orc, mode):
    """2 to 255 rows against an aligned N x K operand, where 64 x 64 tiles
    would be few (the chain kernel, 4 rows per block): row counts not a
    multiple of 4, strided A and C."""
    rng = np.random.default_rng(878 + mode)
    for (m, n, k, lda, ldb) in ((2, 33, 64, 64, 64), (3, 100, 260, 263, 264), (5, 16, 128, 130, 132),
                                (8, 517, 1000, 1000, 1004), (16, 4096, 4096, 4096, 4096),
                                (37, 300, 128, 128, 132), (128, 768, 768, 768, 768),
                                (255, 900, 516, 516, 516)):
        A = _mixed(rng, (m, k), 0.01)
        Bt = _mixed(rng, (n, k), 0.001, 0.02)
        say(f"gemm_nt few rows {m}x{n}x{k} lda {lda} ldb {ldb} mode {mode}")
        got, flatC = _nt_gpu(A, Bt, mode, lda, ldb, n + 5, (1, 0, 2))
        assert_same_bits(got, _nt_oracle(orc, A, Bt, mode), f"nt few rows {m}x{n}x{k} mode {mode}")
        _check_gaps(flatC, m, n, n + 5, 2)


@pytest.mark.parametrize("mode", MODES)
def test_single_column_streamed(orc, mode):
    """n = 1 with aligned rows of A, B and C contiguous, k > 512: the column
    streamed against the rows of A through the chain kernel."""
    rng = np.random.default_rng(885 + mode)
    for (m, k, lda) in ((1, 516, 516), (17, 1000, 1004), (333, 700, 704), (4096, 4096, 4096)):
        A = _mixed(rng, (m, k), 0.002, 0.02)
        B = _mixed(rng, (k, 1), 0.01)
        say(f"gemm single column (streamed) {m}x1x{k} lda {lda} mode {mode}")
        dA, _ = to_device_strided(A, lda, 0)
        dB = torch().from_numpy(B).cuda()
        got = to_host(og.gemm(dA, dB, mode))
        assert_same_bits(got, orc.gemm(A, B, mode), f"streamed {m}x1x{k} mode {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_single_column(orc, mode):
    """n = 1: the rows of A against one column of B (strided), every output;
    rows 16-byte aligned or not, k not a multiple of 16, k = 0."""
    rng = np.random.default_rng(880 + mode)
    for (m, k, lda, ldb, ldc, offA) in ((1, 1, 1, 1, 1, 0), (70, 33, 33, 1, 1, 0),
                                        (64, 64, 64, 3, 2, 0), (65, 128, 128, 1, 1, 4),
                                        (300, 517, 520, 7, 5, 1), (240, 960, 960, 1, 1, 0),
                                        (1000, 0, 1, 1, 1, 0), (4096, 4096, 4096, 1, 1, 0)):
        A = _mixed(rng, (m, k), 0.002, 0.02)
        B = _mixed(rng, (k, 1), 0.01)
        say(f"gemm single column {m}x1x{k} lda {lda} ldb {ldb} mode {mode}")
        dA, _ = to_device_strided(A, lda, offA)
        dB, _ = to_device_strided(B, ldb, 2)
        fill = np.full((m, 1), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
        dC, flatC = to_device_strided(fill, ldc, 1, gap_bits=synth.GAP_OUT_BITS)
        og.gemm(dA, dB, mode, out=dC)
        got = to_host(dC)
        assert_same_bits(got, orc.gemm(A, B, mode), f"{m}x1x{k} mode {mode}")
        _check_gaps(to_host(flatC), m, 1, ldc, 1)


def test_single_column_variants_agree(orc):
    """The tile kernels on an n = 1 product give the row-dot kernel's bits."""
    rng = np.random.default_rng(890)
    A = _mixed(rng, (333, 700), 0.01)
    B = _mixed(rng, (700, 1), 0.01)
    dA, dB = torch().from_numpy(A).cuda(), torch().from_numpy(B).cuda()
    for mode in MODES:
        want = orc.gemm(A, B, mode)
        for variant in (0, 1, 4, 6, 10, 12, 14):
            og.set_variant(variant)
            say(f"gemm single column variant {variant} mode {mode}")
            assert_same_bits(to_host(og.gemm(dA, dB, mode)), want,
                             f"single column variant {variant} mode {mode}")
        og.set_variant(0)


@pytest.mark.parametrize("batch", [1, 8])
def test_squeeze_excitation_convs(orc, batch):
    """The 16 squeeze-and-excitation convolutions of MobileNetV3-large (1x1 on
    a 1x1 input; at batch 1 single-column products), plus a grouped one."""
    shapes = synth.mobilenetv3_large_se(batch) + [
        synth.ConvShape("se_grouped", batch, 96, 1, 1, 40, 1, 1, groups=4),
        synth.ConvShape("se_odd", batch, 37, 1, 1, 65, 1, 1)]
    for i, s in enumerate(shapes):
        x, w = synth.conv_inputs(s, synth.seed_for(7, 50 * batch + i))
        w = w.copy()
        synth.inject_specials(w.reshape(w.shape[0], -1), 0.002, i)
        for mode in MODES:
            say(f"se conv {s} mode {mode}")
            t = torch()
            y = og.conv2d(t.from_numpy(x).cuda(), t.from_numpy(w).cuda(), groups=s.groups,
                          mode=mode)
            want = orc.conv2d(x, w, mode, groups=s.groups)
            assert_same_bits(to_host(y), want, f"{s} mode {mode}")
