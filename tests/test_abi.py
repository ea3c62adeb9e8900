"""The C-ABI library on a host without a GPU: it loads, exports every symbol
``include/og.h`` declares, and rejects invalid arguments before touching the
device.  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "og.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(og_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return og.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"og_gemm_f32", "og_conv2d_f32", "og_conv2d_f32_ex", "og_set_stream",
            "og_last_error"} <= set(names)
    for name in names:
        assert hasattr(L, name), f"{name} is declared in og.h but not exported"


def test_version(L):
    assert re.fullmatch(r"\d+\.\d+\.\d+", og.version())


NULL = None
P = ctypes.c_void_p(16)  # a non-null pointer that is never dereferenced (arguments fail first)


@pytest.mark.parametrize("args,why", [
    ((4, 4, 4, P, 4, P, 4, P, 4, 7), "mode"),
    ((-1, 4, 4, P, 4, P, 4, P, 4, 0), "negative m"),
    ((4, -1, 4, P, 4, P, 4, P, 4, 0), "negative n"),
    ((4, 4, -1, P, 4, P, 4, P, 4, 0), "negative k"),
    ((4, 4, 5, P, 4, P, 4, P, 4, 0), "lda < k"),
    ((4, 5, 4, P, 4, P, 4, P, 5, 0), "ldb < n"),
    ((4, 5, 4, P, 4, P, 5, P, 4, 1), "ldc < n"),
    ((4, 4, 4, NULL, 4, P, 4, P, 4, 0), "A null"),
    ((4, 4, 4, P, 4, NULL, 4, P, 4, 0), "B null"),
    ((4, 4, 4, P, 4, P, 4, NULL, 4, 1), "C null"),
    ((4, 4, 0, P, 0, P, 4, P, 4, 0), "lda must be >= 1 even for k = 0"),
])
def test_gemm_rejects_before_launch(L, args, why):
    assert L.og_gemm_f32(*args) == og.OG_ERR_INVALID_ARG, why
    assert L.og_last_error()


@pytest.mark.parametrize("args,why", [
    ((4, 4, 4, P, 4, P, 4, P, 4, 3), "mode"),
    ((-1, 4, 4, P, 4, P, 4, P, 4, 0), "negative m"),
    ((4, 4, 5, P, 4, P, 5, P, 4, 0), "lda < k"),
    ((4, 5, 6, P, 6, P, 5, P, 5, 0), "ldb < k (B is n x k)"),
    ((4, 5, 4, P, 4, P, 4, P, 4, 1), "ldc < n"),
    ((4, 4, 4, P, 4, NULL, 4, P, 4, 0), "B null"),
    ((4, 4, 4, P, 4, P, 4, NULL, 4, 1), "C null"),
])
def test_gemm_nt_rejects_before_launch(L, args, why):
    assert L.og_gemm_nt_f32(*args) == og.OG_ERR_INVALID_ARG, why
    assert L.og_last_error()


def test_gemm_nt_ldb_is_checked_against_k_not_n(L):
    """n = 9 > ldb = 5 >= k: valid arguments, so with no GPU the call gets as far
    as the device check."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert L.og_gemm_nt_f32(2, 9, 5, P, 5, P, 5, P, 9, 0) == og.OG_ERR_DEVICE
    assert L.og_gemm_nt_f32(0, 9, 5, NULL, 5, NULL, 5, NULL, 9, 0) == og.OG_OK


def test_gemm_empty_is_a_no_op(L):
    assert L.og_gemm_f32(0, 4, 4, NULL, 4, NULL, 4, NULL, 4, 0) == og.OG_OK
    assert L.og_gemm_f32(3, 0, 4, NULL, 4, NULL, 1, NULL, 1, 1) == og.OG_OK
    assert L.og_last_error() == b""


def test_too_large(L):
    assert L.og_gemm_f32(1 << 31, 1, 1, P, 1, P, 1, P, 1, 0) == og.OG_ERR_TOO_LARGE


def _conv(L, N=1, Cin=4, H=5, W=5, Cout=4, G=1, KH=3, KW=3, s=(1, 1), p=(0, 0, 0, 0), d=(1, 1),
          x=P, w=P, y=P, mode=0):
    return L.og_conv2d_f32_ex(N, Cin, H, W, Cout, G, KH, KW, s[0], s[1], p[0], p[1], p[2], p[3],
                              d[0], d[1], x, w, y, mode)


@pytest.mark.parametrize("kw,why", [
    (dict(mode=3), "mode"),
    (dict(N=0), "N"), (dict(Cin=0), "Cin"), (dict(H=0), "H"), (dict(KW=0), "KW"),
    (dict(G=3), "Cin % G"), (dict(Cin=6, G=3, Cout=4), "Cout % G"),
    (dict(s=(0, 1)), "stride"), (dict(d=(1, 0)), "dilation"), (dict(p=(0, -1, 0, 0)), "pad"),
    (dict(KH=7), "window larger than the input"),
    (dict(x=NULL), "x null"), (dict(w=NULL), "w null"), (dict(y=NULL), "y null"),
])
def test_conv_rejects_before_launch(L, kw, why):
    assert _conv(L, **kw) == og.OG_ERR_INVALID_ARG, why
    assert L.og_last_error()


def _conv_epi(L, act=0, bias=NULL, residual=NULL, **kw):
    a = dict(N=1, Cin=4, H=5, W=5, Cout=4, G=1, KH=3, KW=3, s=(1, 1), p=(0, 0, 0, 0),
             d=(1, 1), x=P, w=P, y=P, mode=0)
    a.update(kw)
    return L.og_conv2d_f32_epi(a["N"], a["Cin"], a["H"], a["W"], a["Cout"], a["G"], a["KH"],
                               a["KW"], a["s"][0], a["s"][1], a["p"][0], a["p"][1], a["p"][2],
                               a["p"][3], a["d"][0], a["d"][1], a["x"], a["w"], bias, act,
                               residual, a["y"], a["mode"])


@pytest.mark.parametrize("kw,why", [
    (dict(act=2), "activation"), (dict(act=-1), "activation"), (dict(act=1, mode=3), "mode"),
    (dict(bias=P, N=0), "N"), (dict(residual=P, y=NULL), "y null"),
    (dict(act=1, G=3), "Cin % G"),
])
def test_conv_epilogue_rejects_before_launch(L, kw, why):
    assert _conv_epi(L, **kw) == og.OG_ERR_INVALID_ARG, why
    assert L.og_last_error()


def test_out_size_matches_the_formula():
    orc = oracle.get()
    rng = np.random.default_rng(0)
    for _ in range(2000):
        size, k, stride, pb, pa, dil = (int(v) for v in rng.integers(1, 9, size=6))
        pb -= 1
        pa -= 1
        want = orc.conv_out_size(size, k, stride, pb, pa, dil)
        got = og.conv2d_out_size(size, k, stride, pb, pa, dil)
        assert (got if got >= 1 else 0) == (want if want >= 1 else 0), (size, k, stride, pb, pa,
                                                                        dil)


def test_variant_and_stream_state(L):
    assert L.og_set_variant(34) == og.OG_ERR_INVALID_ARG
    assert L.og_set_variant(33) == og.OG_OK
    assert L.og_set_variant(-1) == og.OG_ERR_INVALID_ARG
    assert L.og_set_variant(3) == og.OG_OK and L.og_get_variant() == 3
    assert L.og_set_variant(0) == og.OG_OK
    assert L.og_set_stream(None) == og.OG_OK and L.og_get_stream() is None


def test_no_device_is_reported_not_hidden(L):
    """With valid arguments and no usable gfx950 device, the call reports
    OG_ERR_DEVICE (there is no CPU fallback)."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    assert L.og_gemm_f32(2, 2, 2, P, 2, P, 2, P, 2, 0) == og.OG_ERR_DEVICE


def test_conv_too_many_taps_is_too_large(L):
    """K = Cin/G*KH*KW above 2^22 is refused before any launch: the kernels
    address a tile's weight rows (row stride K) with 32-bit byte offsets."""
    # 2^20 channels x 3x3 window: K = 9 * 2^20 > 2^22, the input only 9 * 2^20 elements
    assert _conv(L, Cin=1 << 20, Cout=2, H=3, W=3) == og.OG_ERR_TOO_LARGE
    assert b"2^22" in L.og_last_error()
    # grouped: K per group = 9 * 2^19 > 2^22 too; with four groups 9 * 2^18 fits
    assert _conv(L, Cin=1 << 20, Cout=4, G=2, H=3, W=3) == og.OG_ERR_TOO_LARGE
    assert _conv(L, Cin=1 << 20, Cout=4, G=4, H=3, W=3) != og.OG_ERR_TOO_LARGE
    # K = 2^22 exactly is accepted (with no GPU the call then stops at the device check)
    try:
        import torch
        gpu = torch.cuda.is_available()
    except ImportError:
        gpu = False
    if not gpu:
        assert _conv(L, Cin=1 << 22, Cout=1, H=1, W=1, KH=1, KW=1) == og.OG_ERR_DEVICE


def test_binding_row_stride_of_views():
    """The binding's row stride: a view with several columns must have unit
    column stride whatever its number of rows, including a single row taken
    from a column slice (its columns are a row of the parent apart)."""
    import torch
    Y = torch.zeros(8, 6)
    assert og._ld(Y) == 6
    assert og._ld(Y[2:3]) == 6                      # one contiguous row
    assert og._ld(Y[:, 1:4]) == 6                   # rows of a column slice
    assert og._ld(Y[:, 2:3]) == 6                   # one column: stride(1) unused
    assert og._ld(Y[:, 2].unsqueeze(1)) == 6
    assert og._ld(torch.zeros(1, 0)) == 1
    for bad in (Y[:, 2].unsqueeze(0),               # a column as a (1, 8) row: stride(1) = 6
                Y.t(),                              # a transposed view
                Y[:, ::2],                          # every other column
                Y.t()[:1]):                         # a single row of a transposed view
        with pytest.raises(ValueError):
            og._ld(bad)


@pytest.mark.parametrize("variant", [21, 22, 23, 24, 25])
def test_split_variants_refused_in_exact_and_fast(L, variant):
    """A split-k variant forced in exact or fast mode is reported as
    OG_ERR_NOT_EXACT before anything is queued ("Exact mode": an operator
    without an exact kernel says so instead of approximating)."""
    assert L.og_set_variant(variant) == og.OG_OK
    try:
        for mode in (og.EXACT, og.FAST):
            assert L.og_gemm_f32(4, 4, 4, P, 4, P, 4, P, 4, mode) == og.OG_ERR_NOT_EXACT
            assert b"split-k" in L.og_last_error()
            assert L.og_gemm_nt_f32(4, 4, 4, P, 4, P, 4, P, 4, mode) == og.OG_ERR_NOT_EXACT
            assert _conv(L, mode=mode) == og.OG_ERR_NOT_EXACT
            assert _conv_epi(L, act=1, mode=mode) == og.OG_ERR_NOT_EXACT
        # in mode 2 the same call passes the checks (and, with no GPU, stops at the device)
        try:
            import torch
            gpu = torch.cuda.is_available()
        except ImportError:
            gpu = False
        if not gpu:
            assert L.og_gemm_f32(4, 4, 4, P, 4, P, 4, P, 4, og.FAST_MFMA) == og.OG_ERR_DEVICE
    finally:
        L.og_set_variant(0)


# The automatic choice for a product depends on the shape and mode alone, so
# it is host logic: og_gemm_choice reports it without a device.
def test_gemm_choice_of_the_4096_product(L):
    # the 256 x 256 tile with eight waves: the kernel whose launch time and
    # HBM counters the 4096^3 fast-mode measurement reports
    assert og.gemm_choice(4096, 4096, 4096, "fast") == 17


@pytest.mark.parametrize("m,n,k", [(512, 11008, 4096), (1, 4096, 4096), (8, 4096, 4096),
                                   (1000, 777, 1531), (256, 256, 256), (64, 3136, 64),
                                   (2048, 8192, 8192)])
def test_gemm_choice_is_a_variant_of_its_mode(L, m, n, k):
    tiles = set(range(2, 18)) | {20}
    assert og.gemm_choice(m, n, k, "fast") in tiles | {29, 30}
    assert og.gemm_choice(m, n, k, "exact") in tiles - {9, 14, 15, 16}
    assert og.gemm_choice(m, n, k, "fast_mfma") in tiles | {21, 22, 23, 24, 25, 29, 30}


def test_gemm_choice_mode2_splits_a_short_product(L):
    # 256^3 is bound by its k chain: mode 2 splits k
    assert og.gemm_choice(256, 256, 256, "fast_mfma") in (21, 22, 23, 24, 25)


@pytest.mark.parametrize("args,status", [
    ((4, 4, 4, 7), og.OG_ERR_INVALID_ARG),
    ((0, 4, 4, 0), og.OG_ERR_INVALID_ARG),
    ((4, 1, 4, 1), og.OG_ERR_INVALID_ARG),
    ((4, 4, 0, 1), og.OG_ERR_INVALID_ARG),
    ((2 ** 31, 4, 4, 1), og.OG_ERR_TOO_LARGE),
])
def test_gemm_choice_rejects(L, args, status):
    assert L.og_gemm_choice(*args) == status
    assert L.og_last_error()
