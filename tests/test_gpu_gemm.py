"""GPU parity of the matrix product: libog (through its C ABI) against the CPU
oracle, bit for bit, in exact and fast mode.

Sizes: every dimension swept over 0..70 with the others fixed (the sweep the
exact-mode page describes under "Checking it"), random row strides and
pointer offsets, special values; and every full-size workload with every
output compared, in the launch configuration the benchmark times: 256^3,
4096^3 and the ragged 1000x777x1531 with row strides dim+13 (each with 0.1 %
special values and as a clean copy), the prefill shape and the skinny m = 1
shape.  For those the SHA-256 of the GPU's outputs, of the oracle's and the
stored one (tests/golden/full_size_sha256.json) are printed at the end of
the session and must all be equal.
"""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import full_size
import oracle
import synth
from gpu_util import (assert_same_bits, bits, record_hashes, say, to_device_strided, to_host,
                      torch)

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


def _mixed(rng, shape, special_frac):
    """N(0,1) values with a fraction of special values (NaN kinds, +-inf, subnormal, -0)."""
    v = rng.standard_normal(shape).astype(np.float32)
    if special_frac > 0 and v.size:
        synth.inject_specials(v.reshape(shape[0], -1), special_frac, int(rng.integers(1 << 30)))
    return v


def _run_gpu(A, B, mode, lda, ldb, ldc, offs=(0, 0, 0)):
    m, k = A.shape
    n = B.shape[1]
    dA, _ = to_device_strided(A, lda, offs[0])
    dB, _ = to_device_strided(B, ldb, offs[1])
    fill = np.full((m, n), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
    dC, flatC = to_device_strided(fill, ldc, offs[2], gap_bits=synth.GAP_OUT_BITS)
    og.gemm(dA, dB, mode, out=dC)
    torch().cuda.synchronize()
    return to_host(dC), to_host(flatC)


def _check_gaps(flatC, m, n, ldc, off):
    u = flatC.view(np.uint32)
    mask = np.ones(u.shape, bool)
    if m and n:
        idx = off + np.arange(m)[:, None] * ldc + np.arange(n)[None, :]
        mask[idx.ravel()] = False
    assert np.all(u[mask] == synth.GAP_OUT_BITS), "an element outside C was written"


def _full_gemm(orc, name):
    """Every output of a full-size workload, both modes, against the oracle;
    the gaps of C's row stride untouched; a second run gives the same bits;
    the digests of GPU, oracle and stored values equal."""
    c = full_size.gemm_case(name)
    stored = full_size.stored()[name]
    dA, _ = to_device_strided(c.A, c.lda)
    dB, _ = to_device_strided(c.B, c.ldb)
    for mname, mode in full_size.MODES.items():
        say(f"gemm {name} {c.m}x{c.n}x{c.k} mode {mname}")
        fill = np.full((c.m, c.n), synth.GAP_OUT_BITS, np.uint32).view(np.float32)
        dC, flatC = to_device_strided(fill, c.ldc, 0, gap_bits=synth.GAP_OUT_BITS)
        og.gemm(dA, dB, mode, out=dC)
        got = to_host(dC)
        _check_gaps(to_host(flatC), c.m, c.n, c.ldc, 0)
        say(f"oracle {name} mode {mname}")
        want = full_size.oracle_gemm(orc, c, mode)
        dg, do = full_size.Digest().add(got).hex(), full_size.Digest().add(want).hex()
        record_hashes(name, mname, dg, do, stored[mname])
        assert_same_bits(got, want, f"{name} mode {mname}")
        assert do == stored[mname], f"{name} {mname}: the oracle's digest differs from the stored one"
        og.gemm(dA, dB, mode, out=dC)
        assert np.array_equal(bits(to_host(dC)), bits(got)), f"{name} {mname}: second run differs"
        del dC, flatC


def test_square_256_exact_config(orc):
    """m = n = k = 256, uniform[-1,1] from seed 0: bit for bit, exact and fast."""
    _full_gemm(orc, "gemm_256")


SWEEP = [(d, 37, 45) for d in range(71)] + [(19, d, 45) for d in range(71)] + \
        [(19, 37, d) for d in range(71)]


@pytest.mark.parametrize("mode", MODES)
def test_size_sweep_0_to_70(orc, mode):
    """Every size 0..70 in each dimension, random strides, offsets and special values."""
    rng = np.random.default_rng(100 + mode)
    say(f"gemm sweep mode {mode}")
    for (m, n, k) in SWEEP:
        A = _mixed(rng, (m, k), 0.02)
        B = _mixed(rng, (k, n), 0.02)
        lda = max(1, k) + int(rng.integers(0, 5))
        ldb = max(1, n) + int(rng.integers(0, 5))
        ldc = max(1, n) + int(rng.integers(0, 5))
        offs = tuple(int(o) for o in rng.integers(0, 7, size=3))
        got, flatC = _run_gpu(A, B, mode, lda, ldb, ldc, offs)
        want = orc.gemm(A, B, mode)
        assert_same_bits(got, want, f"sweep {m}x{n}x{k} mode {mode}")
        _check_gaps(flatC, m, n, ldc, offs[2])


@pytest.mark.parametrize("specials", [True, False])
def test_ragged_ld13_full(orc, specials):
    """1000x777x1531 with row strides dim+13 and 0.1% special values: every output."""
    _full_gemm(orc, "gemm_ragged_" + ("specials" if specials else "clean"))


@pytest.mark.parametrize("variant", list(range(1, 21)))
def test_variants_agree(orc, variant):
    """Every kernel variant gives the oracle's bits (no dependence on tiles)."""
    rng = np.random.default_rng(7)
    m, n, k = 131, 301, 97
    A = _mixed(rng, (m, k), 0.01)
    B = _mixed(rng, (k, n), 0.01)
    og.set_variant(variant)
    for mode in MODES:
        say(f"gemm variant {variant} mode {mode}")
        got, _ = _run_gpu(A, B, mode, k + 3, n + 1, n + 2, (1, 2, 3))
        assert_same_bits(got, orc.gemm(A, B, mode), f"variant {variant} mode {mode}")
    # several tiles of the largest tile shapes, each ending inside the problem
    m, n, k = 300, 520, 40
    A = _mixed(rng, (m, k), 0.01)
    B = _mixed(rng, (k, n), 0.01)
    for mode in MODES:
        say(f"gemm variant {variant} {m}x{n}x{k} mode {mode}")
        got, _ = _run_gpu(A, B, mode, k, n, n)
        assert_same_bits(got, orc.gemm(A, B, mode), f"variant {variant} {m}x{n}x{k} mode {mode}")


@pytest.mark.parametrize("variant", [10, 11, 12, 13, 14, 15, 16])
def test_chain_kernel_lengths(orc, variant):
    """The chain kernel over k from 0 to several chunks, with ragged tails,
    rows and columns that end inside a tile, and special values."""
    rng = np.random.default_rng(70 + variant)
    og.set_variant(variant)
    for m, n, k in ((5, 70, 0), (5, 70, 1), (9, 33, 64), (9, 33, 65), (3, 130, 517),
                    (1, 301, 300), (6, 17, 129)):
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        for mode in MODES:
            say(f"gemm chain variant {variant} {m}x{n}x{k} mode {mode}")
            got, _ = _run_gpu(A, B, mode, k + 1, n + 3, n, (0, 1, 0))
            assert_same_bits(got, orc.gemm(A, B, mode), f"chain {variant} {m}x{n}x{k} mode {mode}")
    # B rows 16-byte aligned (ldb and n multiples of 4): the 16-byte producer loads
    for m, n, k, ldb in ((5, 64, 200, 68), (3, 132, 517, 136), (1, 48, 64, 48), (6, 16, 1, 20),
                         (7, 64, 1100, 64)):
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        for mode in MODES:
            say(f"gemm chain variant {variant} aligned {m}x{n}x{k} ldb {ldb} mode {mode}")
            got, _ = _run_gpu(A, B, mode, k, ldb, n + 1, (0, 4, 0))
            assert_same_bits(got, orc.gemm(A, B, mode),
                             f"chain {variant} aligned {m}x{n}x{k} mode {mode}")
    # A rows 16-byte aligned (lda and k multiples of 4; k ends inside a chunk): the
    # 16-byte weight loads; the last case (k not a multiple of 4) loads tap by tap
    for m, n, k, lda in ((5, 70, 516, 520), (9, 64, 132, 132), (2, 33, 4, 4), (3, 40, 131, 132)):
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        for mode in MODES:
            say(f"gemm chain variant {variant} A aligned {m}x{n}x{k} lda {lda} mode {mode}")
            got, _ = _run_gpu(A, B, mode, lda, n + 1, n, (0, 0, 0))
            assert_same_bits(got, orc.gemm(A, B, mode),
                             f"chain {variant} A aligned {m}x{n}x{k} mode {mode}")


@pytest.mark.parametrize("variant", [29, 30])
def test_panel_kernel_products(orc, variant):
    """The panel kernel (fast mode) over k from 0 to many 32-step chunks with
    ragged tails, rows and columns ending inside a block, row strides,
    misaligned and aligned rows of A and B, and special values; in exact
    mode the variant runs the automatic choice."""
    rng = np.random.default_rng(90 + variant)
    og.set_variant(variant)
    # rows of A and B not 16-byte aligned: 4-byte loads
    for m, n, k in ((5, 70, 0), (5, 70, 1), (9, 33, 31), (9, 33, 32), (9, 33, 33), (17, 64, 64),
                    (70, 130, 517), (1, 301, 300), (131, 301, 97)):
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        for mode in MODES:
            say(f"gemm panel variant {variant} {m}x{n}x{k} mode {mode}")
            got, flat = _run_gpu(A, B, mode, k + 1, n + 3, n + 2, (0, 1, 1))
            _check_gaps(flat, m, n, n + 2, 1)
            assert_same_bits(got, orc.gemm(A, B, mode), f"panel {variant} {m}x{n}x{k} mode {mode}")
    # B rows 16-byte aligned (16-byte panel loads), A rows too or not
    for m, n, k, lda, ldb in ((5, 64, 200, 200, 68), (33, 132, 517, 520, 136),
                              (64, 128, 96, 96, 128), (7, 64, 1100, 1101, 64), (40, 4, 36, 36, 4)):
        A = _mixed(rng, (m, k), 0.01)
        B = _mixed(rng, (k, n), 0.01)
        for mode in MODES:
            say(f"gemm panel variant {variant} aligned {m}x{n}x{k} lda {lda} ldb {ldb} mode {mode}")
            got, _ = _run_gpu(A, B, mode, lda, ldb, n + 1, (0, 4, 0))
            assert_same_bits(got, orc.gemm(A, B, mode),
                             f"panel {variant} aligned {m}x{n}x{k} mode {mode}")


@pytest.mark.parametrize("specials", [True, False])
def test_4096_cubed_full(orc, specials):
    """4096^3 with 0.1 % special values and as a clean copy: every output."""
    _full_gemm(orc, "gemm_4096_" + ("specials" if specials else "clean"))


def test_prefill_full(orc):
    _full_gemm(orc, "gemm_prefill")


def test_skinny_full(orc):
    _full_gemm(orc, "gemm_skinny")


def test_k_zero_and_empty():
    """k = 0 stores +0 everywhere; m = 0 or n = 0 does nothing."""
    t = torch()
    C = t.full((3, 5), float("nan"), device="cuda")
    A = t.empty((3, 0), device="cuda")
    B = t.empty((0, 5), device="cuda")
    for mode in MODES:
        say(f"gemm k=0 mode {mode}")
        og.gemm(A, B, mode, out=C)
        assert np.all(bits(to_host(C)) == 0)
    og.gemm(t.empty((0, 4), device="cuda"), t.ones((4, 5), device="cuda"), "exact",
            out=t.empty((0, 5), device="cuda"))
    t.cuda.synchronize()


def test_stream_is_honoured(orc):
    """Work goes to the current torch stream and is ordered on it."""
    t = torch()
    rng = np.random.default_rng(9)
    A = rng.standard_normal((300, 200)).astype(np.float32)
    B = rng.standard_normal((200, 400)).astype(np.float32)
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        dA = t.from_numpy(A).cuda()
        dB = t.from_numpy(B).cuda()
        C = og.gemm(dA, dB, "fast")
        got = C.cpu().numpy()
    assert og.lib().og_get_stream() == s.cuda_stream
    assert_same_bits(got, orc.gemm(A, B, 1), "gemm on a side stream")


def test_single_row_views(orc):
    """Single-row operands and outputs taken as views: a contiguous row of a
    larger matrix is used in place; a row whose columns are not adjacent (a
    column of a matrix viewed as a row) is refused before any launch, and the
    caller's tensors are left as they were."""
    t = torch()
    rng = np.random.default_rng(11)
    Y = rng.standard_normal((8, 6)).astype(np.float32)
    Bm = rng.standard_normal((6, 5)).astype(np.float32)
    dY = t.from_numpy(Y).cuda()
    dB = t.from_numpy(Bm).cuda()
    Z = t.full((4, 5), 7.0, device="cuda")
    for mode in MODES:
        say(f"gemm single-row views mode {mode}")
        og.gemm(dY[2:3], dB, mode, out=Z[3:4])
        got = to_host(Z)
        assert_same_bits(got[3:4], orc.gemm(np.ascontiguousarray(Y[2:3]), Bm, mode),
                         f"single row mode {mode}")
        assert np.all(got[:3] == 7.0), "rows outside the output view were written"
    before = to_host(Z).copy()
    col_as_row = dY[:, 2].unsqueeze(0)                   # (1, 8), stride(1) = 6
    with pytest.raises(ValueError):
        og.gemm(col_as_row, t.ones((8, 5), device="cuda"), "fast", out=Z[:1])
    with pytest.raises(ValueError):                      # B (1 x 4) with stride(1) = 5
        og.gemm(t.ones((2, 1), device="cuda"), Z.t()[:1, :4], "fast",
                out=t.empty((2, 4), device="cuda"))
    with pytest.raises(ValueError):                      # out (1 x 4) with stride(1) = 5
        og.gemm(t.ones((1, 3), device="cuda"), t.ones((3, 4), device="cuda"), "fast",
                out=Z.t()[1:2, :])
    t.cuda.synchronize()
    assert np.array_equal(bits(to_host(Z)), bits(before)), "a refused call wrote its output"
