"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each check takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with
  * the hand-worked cases of ``tests/golden/hand_cases.jsonl`` (each with the
    passage of the pages it follows),
  * closed forms: integer-valued inputs whose every partial sum is exact in
    binary32 give the exact integer product (numpy int64 matmul) in both
    modes; convolutions on such inputs equal torch's float64 convolution,
  * first-principles IEEE binary32 arithmetic on exact rationals
    (``tests/ieee32.py``), one rounding per product and per sum (exact mode)
    or per fused multiply-add (fast mode),
  * invariants the pages state: operand order of a product, blocking and
    splitting, im2col against direct convolution, groups and batch as
    separate calls,
  * the accuracy bound of sequential summation (Higham, section 3.1) that
    the fast-mode page quotes.

The same checks run against deliberately broken copies of the oracle
(``test_oracle_mutations.py``) to show that each plausible mistake fails one.
"""
from __future__ import annotations

import json
import os

import numpy as np

import ieee32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.jsonl")
EXACT, FAST = 0, 1
MODES = {"exact": EXACT, "fast": FAST}


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def from_hex(vals, shape) -> np.ndarray:
    u = np.array([int(v, 16) for v in vals], dtype=np.uint32)
    return u.view(np.float32).reshape(shape).copy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    g, w = bits(got).ravel(), bits(want).ravel()
    if not np.array_equal(g, w):
        bad = np.nonzero(g != w)[0]
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} outputs differ; first at {i}: "
                             f"got {g[i]:08x} want {w[i]:08x}")


def load_hand_cases():
    with open(GOLDEN) as f:
        return [json.loads(line) for line in f if line.strip()]


def check_hand_cases(orc):
    for case in load_hand_cases():
        for mname in case["modes"]:
            mode = MODES[mname]
            if case["op"] == "gemm":
                m, n, k = case["m"], case["n"], case["k"]
                A = from_hex(case["A"], (m, k)) if k else np.zeros((m, 0), np.float32)
                B = from_hex(case["B"], (k, n)) if k else np.zeros((0, n), np.float32)
                want = from_hex(case["C"], (m, n))
                for rowwise in (False, True):
                    C = np.full((m, n), np.nan, np.float32)
                    orc.gemm(A, B, mode, out=C, rowwise=rowwise)
                    assert_bits_equal(C, want, f"{case['id']} {mname} rowwise={rowwise}")
            else:
                x = from_hex(case["x"], (case["N"], case["Cin"], case["H"], case["W"]))
                w = from_hex(case["w"], (case["Cout"], case["Cin"] // case["G"], case["KH"],
                                         case["KW"]))
                for route in ("direct", "im2col"):
                    y = orc.conv2d(x, w, mode, groups=case["G"], stride=case["stride"],
                                   pad=case["pad"], dil=case["dil"], route=route)
                    want = from_hex(case["y"], y.shape)
                    assert_bits_equal(y, want, f"{case['id']} {mname} {route}")


def _int_matrix(rng, shape, lo=-8, hi=8):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def check_integer_closed_form(orc):
    """Integer inputs with every partial sum below 2^24: the exact integer product."""
    rng = np.random.default_rng(11)
    for (m, n, k) in [(1, 1, 1), (3, 5, 7), (17, 9, 33), (6, 40, 2), (40, 3, 100), (5, 8, 200)]:
        A = _int_matrix(rng, (m, k))
        B = _int_matrix(rng, (k, n))
        want = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32)
        # -0 cannot appear: an exact-zero sum from +0 is +0
        for mode in (EXACT, FAST):
            for rowwise in (False, True):
                assert_bits_equal(orc.gemm(A, B, mode, rowwise=rowwise), want,
                                  f"integer product {m}x{n}x{k} mode {mode}")
        # inside row-strided buffers with gaps full of NaN
        Ab = np.full((m, k + 3), np.nan, np.float32)
        Bb = np.full((k, n + 5), np.nan, np.float32)
        Cb = np.full((m, n + 2), 7.0, np.float32)
        Ab[:, :k], Bb[:, :n] = A, B
        orc.gemm(Ab[:, :k], Bb[:, :n], EXACT, out=Cb[:, :n])
        assert_bits_equal(Cb[:, :n], want, "integer product, strided")
        assert np.all(Cb[:, n:] == 7.0), "a gap of C was written"


def _mixed_values(rng, size):
    """Finite values across the binary32 range plus a few specials, as bit patterns."""
    kind = rng.integers(0, 10, size=size)
    v = rng.standard_normal(size).astype(np.float32)
    v = np.where(kind == 1, v * np.float32(1e-20), v)      # products reach the subnormals
    v = np.where(kind == 2, v * np.float32(1e-39), v)      # subnormal inputs
    v = np.where(kind == 3, v * np.float32(1e19), v)       # products near overflow
    v = np.where(kind == 4, np.float32(-0.0), v)
    u = v.view(np.uint32).copy()
    u[kind == 5] = 0x7F800000 if rng.random() < 0.5 else 0xFF800000
    u[(kind == 6) & (rng.random(size) < 0.3)] = 0x7FC12345
    return u


def check_ieee_emulation(orc, trials: int = 60, seed: int = 3):
    """Tiny random products against binary32 arithmetic done on exact rationals."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        m, n = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        k = int(rng.integers(0, 14))
        Au = _mixed_values(rng, m * k).reshape(m, k)
        Bu = _mixed_values(rng, k * n).reshape(k, n)
        A, B = Au.view(np.float32), Bu.view(np.float32)
        for mode in (EXACT, FAST):
            got = bits(orc.gemm(A, B, mode))
            for i in range(m):
                for j in range(n):
                    a = [int(x) for x in Au[i, :]]
                    b = [int(x) for x in Bu[:, j]]
                    want = ieee32.dot_exact_mode(a, b) if mode == EXACT else ieee32.dot_fast_mode(a, b)
                    if int(got[i, j]) != want:
                        raise AssertionError(f"ieee emulation trial {t} mode {mode} ({i},{j}): "
                                             f"got {int(got[i, j]):08x} want {want:08x}")


def check_conv_ieee_emulation(orc, trials: int = 12, seed: int = 4):
    """Tiny random convolutions (padding, stride, dilation, groups) on exact rationals."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        G = int(rng.integers(1, 3))
        cin_g, cout_g = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        N, H, W = 1, int(rng.integers(1, 5)), int(rng.integers(1, 5))
        KH, KW = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        sH, sW = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        dH, dW = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        pad = tuple(int(p) for p in rng.integers(0, 3, size=4))
        pT, pL, pB, pR = pad
        OH = (H + pT + pB - dH * (KH - 1) - 1) // sH + 1
        OW = (W + pL + pR - dW * (KW - 1) - 1) // sW + 1
        if OH < 1 or OW < 1:
            continue
        Cin, Cout = G * cin_g, G * cout_g
        xu = _mixed_values(rng, N * Cin * H * W).reshape(N, Cin, H, W)
        wu = _mixed_values(rng, Cout * cin_g * KH * KW).reshape(Cout, cin_g, KH, KW)
        for mode in (EXACT, FAST):
            y = bits(orc.conv2d(xu.view(np.float32), wu.view(np.float32), mode, groups=G,
                                stride=(sH, sW), pad=pad, dil=(dH, dW)))
            assert y.shape == (N, Cout, OH, OW)
            for oc in range(Cout):
                g = oc // cout_g
                for oy in range(OH):
                    for ox in range(OW):
                        a, b = [], []
                        for c in range(cin_g):
                            for ky in range(KH):
                                for kx in range(KW):
                                    iy, ix = oy * sH - pT + ky * dH, ox * sW - pL + kx * dW
                                    inside = 0 <= iy < H and 0 <= ix < W
                                    a.append(int(wu[oc, c, ky, kx]))
                                    b.append(int(xu[0, g * cin_g + c, iy, ix]) if inside else 0)
                        want = (ieee32.dot_exact_mode(a, b) if mode == EXACT
                                else ieee32.dot_fast_mode(a, b))
                        if int(y[0, oc, oy, ox]) != want:
                            raise AssertionError(f"conv ieee trial {t} mode {mode} "
                                                 f"({oc},{oy},{ox}): got "
                                                 f"{int(y[0, oc, oy, ox]):08x} want {want:08x}")


def check_transpose(orc):
    """(A B)^T = B^T A^T bit for bit: each term's product commutes, the order of p is kept."""
    rng = np.random.default_rng(12)
    for (m, n, k) in [(7, 13, 29), (1, 9, 64), (12, 1, 5)]:
        A = rng.standard_normal((m, k)).astype(np.float32)
        B = rng.standard_normal((k, n)).astype(np.float32)
        for mode in (EXACT, FAST):
            C = orc.gemm(A, B, mode)
            Ct = orc.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), mode)
            assert_bits_equal(Ct.T, C, f"transpose {m}x{n}x{k} mode {mode}")


def check_split(orc):
    """Sub-products over row and column ranges, with offsets and strides, give the same bits."""
    rng = np.random.default_rng(13)
    m, n, k = 23, 31, 47
    A = rng.standard_normal((m, k)).astype(np.float32)
    B = rng.standard_normal((k, n)).astype(np.float32)
    for mode in (EXACT, FAST):
        C = orc.gemm(A, B, mode)
        P = np.full((m, n), np.nan, np.float32)
        for r0, r1 in ((0, 5), (5, 17), (17, 23)):
            for c0, c1 in ((0, 1), (1, 20), (20, 31)):
                orc.gemm(A[r0:r1], B[:, c0:c1], mode, out=P[r0:r1, c0:c1])
        assert_bits_equal(P, C, f"split mode {mode}")


def check_rowwise(orc):
    """The loop-interchanged product equals the per-output loop on a size sweep."""
    rng = np.random.default_rng(14)
    sizes = [(d, 5, 6) for d in range(0, 71, 7)] + [(5, d, 6) for d in range(0, 71, 7)] + \
            [(5, 6, d) for d in range(0, 71, 7)]
    for (m, n, k) in sizes:
        Au = _mixed_values(rng, m * k).reshape(m, k)
        Bu = _mixed_values(rng, k * n).reshape(k, n)
        for mode in (EXACT, FAST):
            a = orc.gemm(Au.view(np.float32), Bu.view(np.float32), mode)
            b = orc.gemm(Au.view(np.float32), Bu.view(np.float32), mode, rowwise=True)
            assert_bits_equal(b, a, f"rowwise {m}x{n}x{k} mode {mode}")


def check_higham(orc):
    """|c - r| <= gamma_K * sum|a b| + 1e-30 with r, the sum of |a b| in float64."""
    rng = np.random.default_rng(15)
    u = 2.0 ** -24
    for (m, n, k) in [(8, 8, 10), (6, 7, 300), (4, 5, 3000)]:
        A = rng.standard_normal((m, k)).astype(np.float32)
        B = rng.standard_normal((k, n)).astype(np.float32)
        r = A.astype(np.float64) @ B.astype(np.float64)
        S = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        gamma = k * u / (1 - k * u)
        for mode in (EXACT, FAST):
            c = orc.gemm(A, B, mode).astype(np.float64)
            err = np.abs(c - r)
            assert np.all(err <= gamma * S + 1e-30), f"Higham bound mode {mode} k {k}"
            # the bound is not vacuous: the computed sums are not the float64 sums
            assert np.any(err > 0)


def _torch_conv_f64(x, w, groups, stride, pad, dil):
    import torch
    import torch.nn.functional as F
    pT, pL, pB, pR = pad
    xt = F.pad(torch.from_numpy(x.astype(np.float64)), (pL, pR, pT, pB))
    yt = F.conv2d(xt, torch.from_numpy(w.astype(np.float64)), stride=stride, dilation=dil,
                  groups=groups)
    return yt.numpy()


CONV_INDEX_CASES = [
    # (N, Cin, H, W, Cout, G, KH, KW, stride, pad(t,l,b,r), dil)
    (2, 4, 7, 9, 6, 2, 3, 3, (2, 1), (1, 2, 0, 1), (1, 2)),
    (1, 3, 11, 10, 4, 1, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)),
    (2, 8, 5, 6, 8, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (2, 8, 5, 6, 16, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (1, 6, 1, 20, 4, 1, 1, 5, (1, 1), (0, 2, 0, 2), (1, 1)),
    (3, 8, 9, 9, 8, 4, 3, 3, (2, 2), (2, 2, 2, 2), (2, 2)),
    (2, 5, 8, 8, 7, 1, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)),
    (1, 4, 6, 5, 3, 1, 2, 3, (1, 2), (0, 1, 1, 0), (2, 1)),
    (1, 3, 4, 4, 2, 1, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1)),
]


def check_conv_integer_vs_torch(orc):
    """Integer inputs, every partial sum exact: torch's float64 convolution, both modes."""
    rng = np.random.default_rng(16)
    for (N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil) in CONV_INDEX_CASES:
        x = rng.integers(-3, 4, size=(N, Cin, H, W)).astype(np.float32)
        w = rng.integers(-3, 4, size=(Cout, Cin // G, KH, KW)).astype(np.float32)
        want = _torch_conv_f64(x, w, G, stride, pad, dil).astype(np.float32)
        for mode in (EXACT, FAST):
            for route in ("direct", "im2col"):
                y = orc.conv2d(x, w, mode, groups=G, stride=stride, pad=pad, dil=dil, route=route)
                assert y.shape == want.shape, f"conv shape {y.shape} vs {want.shape}"
                assert_bits_equal(y + np.float32(0.0), want + np.float32(0.0),
                                  f"conv integer {N, Cin, H, W, Cout, G, KH, KW} {route} {mode}")


def check_conv_routes(orc):
    """Direct convolution equals im2col + product bit for bit, special values included."""
    rng = np.random.default_rng(17)
    for (N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil) in CONV_INDEX_CASES:
        x = _mixed_values(rng, N * Cin * H * W).reshape(N, Cin, H, W).view(np.float32)
        w = _mixed_values(rng, Cout * (Cin // G) * KH * KW).reshape(
            Cout, Cin // G, KH, KW).view(np.float32)
        for mode in (EXACT, FAST):
            a = orc.conv2d(x, w, mode, groups=G, stride=stride, pad=pad, dil=dil)
            b = orc.conv2d(x, w, mode, groups=G, stride=stride, pad=pad, dil=dil, route="im2col")
            assert_bits_equal(a, b, f"routes {N, Cin, H, W, Cout, G} mode {mode}")


def check_conv_1x1_is_gemm(orc):
    """A 1x1, stride-1, unpadded convolution is W [Cout,Cin] times x viewed as [Cin, H*W]."""
    rng = np.random.default_rng(18)
    N, Cin, H, W, Cout = 2, 9, 5, 7, 6
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = rng.standard_normal((Cout, Cin, 1, 1)).astype(np.float32)
    for mode in (EXACT, FAST):
        y = orc.conv2d(x, w, mode)
        for n in range(N):
            c = orc.gemm(w.reshape(Cout, Cin), x[n].reshape(Cin, H * W), mode)
            assert_bits_equal(y[n].reshape(Cout, H * W), c, f"1x1 as product mode {mode}")


def check_conv_groups_and_batch(orc):
    """A grouped convolution is G separate ones; a batch is N single-image calls."""
    rng = np.random.default_rng(19)
    N, Cin, H, W, Cout, G = 3, 6, 6, 5, 9, 3
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = rng.standard_normal((Cout, Cin // G, 3, 2)).astype(np.float32)
    kw = dict(stride=(2, 1), pad=(1, 0, 1, 1), dil=(1, 2))
    for mode in (EXACT, FAST):
        y = orc.conv2d(x, w, mode, groups=G, **kw)
        ci, co = Cin // G, Cout // G
        for g in range(G):
            yg = orc.conv2d(np.ascontiguousarray(x[:, g * ci:(g + 1) * ci]),
                            np.ascontiguousarray(w[g * co:(g + 1) * co]), mode, **kw)
            assert_bits_equal(y[:, g * co:(g + 1) * co], yg, f"group {g} mode {mode}")
        for n in range(N):
            yn = orc.conv2d(np.ascontiguousarray(x[n:n + 1]), w, mode, groups=G, **kw)
            assert_bits_equal(y[n:n + 1], yn, f"image {n} mode {mode}")


def check_conv1d_library(orc):
    """A 1-D convolution run as H = 1 equals numpy's correlate on integer inputs."""
    rng = np.random.default_rng(20)
    Cin, Wd, Cout, KW, p = 3, 25, 2, 5, 2
    x = rng.integers(-4, 5, size=(1, Cin, 1, Wd)).astype(np.float32)
    w = rng.integers(-4, 5, size=(Cout, Cin, 1, KW)).astype(np.float32)
    for mode in (EXACT, FAST):
        y = orc.conv2d(x, w, mode, pad=(0, p, 0, p))
        assert y.shape == (1, Cout, 1, Wd + 2 * p - KW + 1)
        for oc in range(Cout):
            want = np.zeros(y.shape[3], np.int64)
            for c in range(Cin):
                xp = np.pad(x[0, c, 0].astype(np.int64), (p, p))
                want += np.correlate(xp, w[oc, c, 0].astype(np.int64), mode="valid")
            assert np.array_equal(y[0, oc, 0].astype(np.int64), want), f"1-D conv oc {oc}"


def check_identity(orc):
    """A = I: C = B with -0 made +0; a special value in a column of B meets 0 in the other rows."""
    rng = np.random.default_rng(21)
    k, n = 9, 11
    B = rng.standard_normal((k, n)).astype(np.float32)
    B[4:, 5:] *= np.float32(1e-39)                       # subnormals
    Bu = B.view(np.uint32)
    Bu[0, 0] = 0x80000000                                # -0
    Bu[1, 1] = 0xFFC00001                                # NaN with payload
    Bu[2, 2] = 0x7F800000                                # +inf
    Bu[3, 3] = 0xFF800000                                # -inf
    eye = np.eye(k, dtype=np.float32)
    want = Bu.copy()
    want[0, 0] = 0
    want[:, 1] = ieee32.QNAN                             # 1*NaN and 0*NaN
    want[:, 2] = ieee32.QNAN                             # 0*inf in every other row
    want[2, 2] = 0x7F800000                              # 1*inf plus finite zeros
    want[:, 3] = ieee32.QNAN
    want[3, 3] = 0xFF800000
    for mode in (EXACT, FAST):
        assert_bits_equal(orc.gemm(eye, B, mode), want.view(np.float32), f"identity mode {mode}")


def check_single_outputs(orc):
    """The one-output helpers (a product's (row, column) outputs, a
    convolution's outputs at flat indices of y [N, Cout, OH, OW]) equal the
    whole oracle's outputs at the same places: every output, in shuffled
    order, of products with row strides and special values, and of
    convolutions whose four output axes have different lengths (so a flat
    index decoded with two axes swapped lands on another output)."""
    rng = np.random.default_rng(21)

    def values(size, special):
        if special:  # mostly non-finite sums: the classes of the specials
            return _mixed_values(rng, size).view(np.float32)
        return rng.standard_normal(size).astype(np.float32)  # exact and fast differ

    for (m, n, k, lda, ldb, special) in ((7, 11, 13, 16, 12, False), (7, 11, 13, 16, 12, True),
                                         (1, 9, 40, 40, 9, False), (5, 1, 3, 7, 2, True)):
        for mode in (EXACT, FAST):
            A = values(m * lda, special).reshape(m, lda)[:, :k]
            B = values(k * ldb, special).reshape(k, ldb)[:, :n]
            full = orc.gemm(A, B, mode)
            order = rng.permutation(m * n)
            rows, cols = order // n, order % n
            got = orc.gemm_at(A, B, rows, cols, mode)
            assert_bits_equal(got, full[rows, cols], f"gemm_at {m}x{n}x{k} mode {mode}")
    for (N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil, special) in (
            (2, 4, 9, 6, 6, 2, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2), False),
            (3, 3, 5, 11, 5, 1, 1, 3, (1, 3), (0, 1, 0, 2), (1, 1), False),
            (2, 4, 9, 6, 6, 2, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2), True)):
        for mode in (EXACT, FAST):
            x = values(N * Cin * H * W, special).reshape(N, Cin, H, W)
            w = values(Cout * (Cin // G) * KH * KW, special).reshape(Cout, Cin // G, KH, KW)
            full = orc.conv2d(x, w, mode, groups=G, stride=stride, pad=pad, dil=dil)
            flat = rng.permutation(full.size)
            got = orc.conv2d_at(x, w, flat, mode, groups=G, stride=stride, pad=pad, dil=dil)
            assert_bits_equal(got, full.ravel()[flat], f"conv2d_at {full.shape} mode {mode}")


def fused_unfused_family(rng, m: int = 300, n: int = 130):
    """A and B whose output (i, j) is c_ij * 1 + a_ij * b_j with
    c_ij = -round(a_ij * b_j) (every other term a product with zero; B's column
    j is 1 at row 2j and b_j at row 2j+1).  Returns A, B and the fused result,
    from first principles: rounded separately the two terms cancel to +0;
    fused, the sum is the rounding error of a*b, exact in float64 (the
    product of two binary32 values has at most 48 significant bits)."""
    k = 2 * n
    a = rng.uniform(1, 2, (m, n)) * np.where(rng.random((m, n)) < .5, 1.0, -1.0)
    a = (a * 2.0 ** rng.integers(-20, 20, (m, n))).astype(np.float32)
    b = rng.uniform(1, 2, n).astype(np.float32)
    exact_prod = a.astype(np.float64) * b.astype(np.float64)
    prod32 = exact_prod.astype(np.float32)  # round to nearest even
    A = np.zeros((m, k), np.float32)
    A[:, 0::2] = -prod32
    A[:, 1::2] = a
    B = np.zeros((k, n), np.float32)
    B[2 * np.arange(n), np.arange(n)] = 1.0
    B[2 * np.arange(n) + 1, np.arange(n)] = b
    err = exact_prod - prod32.astype(np.float64)
    fused = err.astype(np.float32)
    assert np.all(fused.astype(np.float64) == err), "the error of a binary32 product is exact"
    return A, B, fused


def check_fused_unfused_family(orc):
    """Exact mode gives +0 for every c + a*b with c = -round(a*b) placed
    first; fast mode gives the rounding error of a*b ("Exact mode", rule 1:
    no fused multiply-add; "Matrix product and convolution kernels", section
    "Fast mode": one fused multiply-add per term)."""
    A, B, fused = fused_unfused_family(np.random.default_rng(31), 40, 50)
    assert np.count_nonzero(fused) > 0.9 * fused.size
    for rowwise in (False, True):
        assert_bits_equal(orc.gemm(A, B, EXACT, rowwise=rowwise), np.zeros_like(fused),
                          f"exact, rowwise={rowwise}")
        assert_bits_equal(orc.gemm(A, B, FAST, rowwise=rowwise), fused, f"fast, rowwise={rowwise}")


def underflow_family(rng, m: int, n: int, k: int):
    """A = 2^-100 and B = +-(1..2) * 2^-60 (negative in odd columns): every
    product is a non-zero value far below the smallest subnormal.  Rounded
    on its own (exact mode) a product is a signed zero and +0 + (-0) = +0, so
    every output is +0.  Fused with the sum (fast mode), the exact result of
    the first term of an odd column is negative and rounds to -0; every later
    term adds another negative amount to -0, so those outputs are -0 (even
    columns +0).  Returns A, B and the fast-mode bits."""
    A = np.full((m, k), 2.0 ** -100, np.float32)
    B = (rng.uniform(1, 2, (k, n)) * 2.0 ** -60).astype(np.float32)
    B[:, 1::2] *= -1
    fast = np.zeros((m, n), np.uint32)
    if k > 0:
        fast[:, 1::2] = 0x80000000
    return A, B, fast


def check_underflow_sign(orc):
    """IEEE 754 rounding of a fused multiply-add whose exact result is a
    non-zero negative number too small to represent gives -0; a separately
    rounded product and sum give +0 ("Exact mode", rules 1 and 3; "Matrix
    product and convolution kernels", section "Fast mode")."""
    rng = np.random.default_rng(41)
    for k in (1, 2, 7):
        A, B, fast = underflow_family(rng, 3, 6, k)
        for rowwise in (False, True):
            assert np.all(bits(orc.gemm(A, B, EXACT, rowwise=rowwise)) == 0), f"exact k={k}"
            assert np.array_equal(bits(orc.gemm(A, B, FAST, rowwise=rowwise)), fast), f"fast k={k}"


def check_out_size(orc):
    """The output-size formula against torch's output shapes, and the k = 0 and empty cases."""
    for (N, Cin, H, W, Cout, G, KH, KW, stride, pad, dil) in CONV_INDEX_CASES:
        x = np.ones((N, Cin, H, W), np.float32)
        w = np.ones((Cout, Cin // G, KH, KW), np.float32)
        want = _torch_conv_f64(x, w, G, stride, pad, dil).shape
        assert orc.conv_out_size(H, KH, stride[0], pad[0], pad[2], dil[0]) == want[2]
        assert orc.conv_out_size(W, KW, stride[1], pad[1], pad[3], dil[1]) == want[3]
    assert orc.conv_out_size(2, 3, 1, 0, 0, 1) < 1   # kernel larger than the input
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 4), np.float32)
    for mode in (EXACT, FAST):
        C = np.full((3, 4), np.nan, np.float32)
        orc.gemm(A, B, mode, out=C)
        assert np.all(bits(C) == 0), "k = 0 must store +0"
        orc.gemm(np.zeros((0, 5), np.float32), np.ones((5, 4), np.float32), mode)


ALL_CHECKS = [
    check_hand_cases, check_integer_closed_form, check_ieee_emulation, check_conv_ieee_emulation,
    check_transpose, check_split, check_rowwise, check_higham, check_conv_integer_vs_torch,
    check_conv_routes, check_conv_1x1_is_gemm, check_conv_groups_and_batch,
    check_conv1d_library, check_identity, check_out_size, check_single_outputs,
    check_fused_unfused_family, check_underflow_sign,
]
