"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.

Each mutant is ``oracle/ogref.c`` with one textual change, compiled with the
oracle's own flags into a temporary directory.  A mutant passes the test
when at least one pin raises; a mutant no pin notices would mean the pins
leave that part of the oracle unchecked.
"""
import os

import pytest

import oracle
import pins

MUTANTS = [
    # (name, text in ogref.c, replacement)
    ("terms_in_decreasing_p",
     "for (int64_t p = 0; p < k; p++)\n        acc = add_term(",
     "for (int64_t p = k - 1; p >= 0; p--)\n        acc = add_term("),
    ("last_term_dropped",
     "for (int64_t p = 0; p < k; p++)\n        acc = add_term(",
     "for (int64_t p = 0; p + 1 < k; p++)\n        acc = add_term("),
    ("exact_mode_fused",
     "float prod = a * b;\n    acc = acc + prod;",
     "acc = fmaf(a, b, acc);"),
    ("fast_mode_unfused",
     "return fmaf(a, b, acc);",
     "return acc + a * b;"),
    ("nan_not_canonical",
     "return isnan(acc) ? canonical_nan() : acc;",
     "return acc;"),
    ("start_from_minus_zero",
     "    float acc = 0.0f;\n    for (int64_t p = 0;",
     "    float acc = -0.0f;\n    for (int64_t p = 0;"),
    ("row_stride_ignored",
     "gemm_one(k, A + i * lda, B, ldb, j, mode);",
     "gemm_one(k, A + i * k, B, ldb, j, mode);"),
    ("conv_kx_before_ky",
     "for (int64_t ky = 0; ky < s->KH; ky++)\n            for (int64_t kx = 0; kx < s->KW; kx++) {",
     "for (int64_t kx = 0; kx < s->KW; kx++)\n            for (int64_t ky = 0; ky < s->KH; ky++) {"),
    ("conv_padding_taps_skipped",
     "                const float wt = w[((oc * cin_g + c) * s->KH + ky) * s->KW + kx];\n"
     "                acc = add_term(acc, wt, v, mode);",
     "                const float wt = w[((oc * cin_g + c) * s->KH + ky) * s->KW + kx];\n"
     "                if (!(iy >= 0 && iy < s->H && ix >= 0 && ix < s->W)) continue;\n"
     "                acc = add_term(acc, wt, v, mode);"),
    ("conv_pad_sign",
     "const int64_t iy = oy * s->sH - s->pT + ky * s->dH;\n                const int64_t ix",
     "const int64_t iy = oy * s->sH + s->pT + ky * s->dH;\n                const int64_t ix"),
    ("conv_group_offset_dropped",
     "v = x[((n * s->Cin + g * cin_g + c) * s->H + iy) * s->W + ix];\n                const float wt",
     "v = x[((n * s->Cin + c) * s->H + iy) * s->W + ix];\n                const float wt"),
    ("conv_dilation_ignored",
     "const int64_t ix = ox * s->sW - s->pL + kx * s->dW;\n                float v",
     "const int64_t ix = ox * s->sW - s->pL + kx;\n                float v"),
    ("conv_width_stride_from_height",
     "const int64_t ix = ox * s->sW - s->pL + kx * s->dW;\n                float v",
     "const int64_t ix = ox * s->sH - s->pL + kx * s->dW;\n                float v"),
    ("out_size_off_by_one",
     "return floor_div(size + pad_before + pad_after - dil * (k - 1) - 1, stride) + 1;",
     "return floor_div(size + pad_before + pad_after - dil * (k - 1), stride) + 1;"),
    ("rowwise_from_minus_zero",
     "                acc[j] = 0.0f;",
     "                acc[j] = -0.0f;"),
    ("gemm_at_mode_ignored",
     "out[t] = gemm_one(k, A + rows[t] * lda, B, ldb, cols[t], mode);",
     "out[t] = gemm_one(k, A + rows[t] * lda, B, ldb, cols[t], MODE_EXACT);"),
    ("conv_at_row_and_column_swapped",
     "out[t] = conv_one(&s, x, w, n, oc, oy, ox, mode);",
     "out[t] = conv_one(&s, x, w, n, oc, ox, oy, mode);"),
    ("conv_at_image_and_channel_swapped",
     "        const int64_t oc = r % s.Cout;\n        const int64_t n = r / s.Cout;",
     "        const int64_t n = r % s.N;\n        const int64_t oc = r / s.N;"),
    ("im2col_rows_kx_major",
     "const int64_t row = (c * s.KH + ky) * s.KW + kx;",
     "const int64_t row = (c * s.KW + kx) * s.KH + ky;"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site of {name} not found exactly once"
    src = tmp_path / "ogref.c"
    src.write_text(source.replace(old, new))
    lib = oracle.compile_lib(str(src), str(tmp_path / f"libogref_{name}.so"))
    mutant = oracle.Oracle(lib, selftest=False)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError) as e:
            caught.append(f"{check.__name__}: {str(e)[:80]}")
    assert caught, f"no pin catches the mutant {name}"


def test_unmutated_copy_passes(tmp_path, source):
    src = tmp_path / "ogref.c"
    src.write_text(source)
    lib = oracle.compile_lib(str(src), str(tmp_path / "libogref_copy.so"))
    copy = oracle.Oracle(lib)
    for check in pins.ALL_CHECKS:
        check(copy)
    assert os.path.exists(lib)
