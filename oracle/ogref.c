/*
 * ogref.c -- the CPU oracle: plain, slow, obviously correct.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU path includes, links or
 * calls this file; the GPU library shares no code with it.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (no -ffast-math / -Ofast, so no flush-to-zero from crtfastmath, and no
 * contraction of a*b+c into a fused operation).  Binary32 on x86-64 uses SSE
 * scalar arithmetic: every float operation is rounded to binary32 on its own,
 * round-to-nearest-even, subnormals kept.
 *
 * What it computes (the pages' own definitions, restated):
 *  - OneModel "Exact mode", section "Matrix product": for each output an
 *    accumulator starting at +0 receives, for p = 0..k-1 in increasing order,
 *    the product A[i][p]*B[p][j] rounded to binary32, and the sum is rounded
 *    to binary32 after each addition; a NaN result is stored as 0x7FC00000;
 *    k = 0 gives +0.
 *  - OneModel "Exact mode", section "Convolution": output (n, oc, y, x) of
 *    group g = oc / (Cout/G) sums over c, then ky, then kx the products
 *    weight[oc][c][ky][kx] * v, v being the input at row y*strideH - padTop +
 *    ky*dilH and column x*strideW - padLeft + kx*dilW of plane g*Cin/G + c, or
 *    +0 outside the plane (still multiplied); canonical NaN; no bias.
 *  - OneModel "Matrix product and convolution kernels", section "Fast mode",
 *    and "Convolution (fast mode)", section "What each output is": the same
 *    order, one accumulator from +0, one fused multiply-add per term
 *    (C99 fmaf, correctly rounded).  The NaN payload, left open by the page,
 *    is made canonical as in exact mode.
 *  - The im2col route (OneModel "Matrix product and convolution kernels",
 *    section "Convolution"): per image and group a (Cin/G*KH*KW) x (OH*OW)
 *    matrix with rows ordered channel, kernel row, kernel column, multiplied
 *    by the group's weight rows with the matrix product above (in its
 *    loop-interchanged form, which keeps every output's order).
 */
#include "ogref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MODE_EXACT 0
#define MODE_FAST 1

/* The quiet NaN with bits 0x7FC00000 (exact-mode rule 4). */
static float canonical_nan(void)
{
    uint32_t u = 0x7FC00000u;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* One term, exact mode: the product rounded, then the sum rounded. */
static float add_term_exact(float acc, float a, float b)
{
    float prod = a * b;
    acc = acc + prod;
    return acc;
}

/* One term, fast mode: a single fused multiply-add. */
static float add_term_fast(float acc, float a, float b)
{
    return fmaf(a, b, acc);
}

static float add_term(float acc, float a, float b, int mode)
{
    return mode == MODE_EXACT ? add_term_exact(acc, a, b) : add_term_fast(acc, a, b);
}

/* The value an output stores: NaN made canonical, everything else as is. */
static float store_value(float acc)
{
    return isnan(acc) ? canonical_nan() : acc;
}

static int valid_mode(int mode)
{
    return mode == MODE_EXACT || mode == MODE_FAST;
}

static int gemm_args_ok(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                        const float *B, int64_t ldb, const float *C, int64_t ldc, int mode)
{
    if (!valid_mode(mode) || m < 0 || n < 0 || k < 0)
        return 0;
    if (lda < (k > 1 ? k : 1) || ldb < (n > 1 ? n : 1) || ldc < (n > 1 ? n : 1))
        return 0;
    if (m > 0 && n > 0 && C == NULL)
        return 0;
    if (m > 0 && n > 0 && k > 0 && (A == NULL || B == NULL))
        return 0;
    return 1;
}

/* One output of the matrix product, the definition written out. */
static float gemm_one(int64_t k, const float *a_row, const float *B, int64_t ldb, int64_t j,
                      int mode)
{
    float acc = 0.0f;
    for (int64_t p = 0; p < k; p++)
        acc = add_term(acc, a_row[p], B[p * ldb + j], mode);
    return store_value(acc);
}

int ogref_gemm_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float *C, int64_t ldc, int mode)
{
    if (!gemm_args_ok(m, n, k, A, lda, B, ldb, C, ldc, mode))
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            C[i * ldc + j] = gemm_one(k, A + i * lda, B, ldb, j, mode);
    return 0;
}

int ogref_gemm_f32_rowwise(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                           const float *B, int64_t ldb, float *C, int64_t ldc, int mode)
{
    if (!gemm_args_ok(m, n, k, A, lda, B, ldb, C, ldc, mode))
        return -1;
    if (m == 0 || n == 0)
        return 0;
    int failed = 0;
#pragma omp parallel
    {
        float *acc = (float *)malloc((size_t)n * sizeof(float));
        if (acc == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < m; i++) {
            if (acc == NULL)
                continue;
            for (int64_t j = 0; j < n; j++)
                acc[j] = 0.0f;
            for (int64_t p = 0; p < k; p++) {
                const float a = A[i * lda + p];
                const float *brow = B + p * ldb;
                if (mode == MODE_EXACT)
                    for (int64_t j = 0; j < n; j++)
                        acc[j] = add_term_exact(acc[j], a, brow[j]);
                else
                    for (int64_t j = 0; j < n; j++)
                        acc[j] = add_term_fast(acc[j], a, brow[j]);
            }
            for (int64_t j = 0; j < n; j++)
                C[i * ldc + j] = store_value(acc[j]);
        }
        free(acc);
    }
    return failed ? -1 : 0;
}

int ogref_gemm_f32_at(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                      const float *B, int64_t ldb, int64_t npts, const int64_t *rows,
                      const int64_t *cols, float *out, int mode)
{
    if (!gemm_args_ok(m, n, k, A, lda, B, ldb, out, n, mode) || npts < 0)
        return -1;
    if (npts > 0 && (rows == NULL || cols == NULL || out == NULL))
        return -1;
    for (int64_t t = 0; t < npts; t++)
        if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npts; t++)
        out[t] = gemm_one(k, A + rows[t] * lda, B, ldb, cols[t], mode);
    return 0;
}

/* floor(a / b) for b > 0 and any sign of a. */
static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b != 0) && (a < 0))
        q -= 1;
    return q;
}

int64_t ogref_conv_out_size(int64_t size, int64_t k, int64_t stride, int64_t pad_before,
                            int64_t pad_after, int64_t dil)
{
    if (stride < 1)
        return 0;
    return floor_div(size + pad_before + pad_after - dil * (k - 1) - 1, stride) + 1;
}

struct conv_shape {
    int64_t N, Cin, H, W, Cout, G, KH, KW, sH, sW, pT, pL, pB, pR, dH, dW, OH, OW;
};

static int conv_shape_init(struct conv_shape *s, int64_t N, int64_t Cin, int64_t H, int64_t W,
                           int64_t Cout, int64_t G, int64_t KH, int64_t KW, int64_t sH,
                           int64_t sW, int64_t pT, int64_t pL, int64_t pB, int64_t pR,
                           int64_t dH, int64_t dW, const float *x, const float *w,
                           const float *y, int mode)
{
    if (!valid_mode(mode))
        return 0;
    if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || G < 1 || KH < 1 || KW < 1)
        return 0;
    if (sH < 1 || sW < 1 || dH < 1 || dW < 1 || pT < 0 || pL < 0 || pB < 0 || pR < 0)
        return 0;
    if (Cin % G != 0 || Cout % G != 0)
        return 0;
    if (x == NULL || w == NULL || y == NULL)
        return 0;
    s->N = N; s->Cin = Cin; s->H = H; s->W = W; s->Cout = Cout; s->G = G;
    s->KH = KH; s->KW = KW; s->sH = sH; s->sW = sW;
    s->pT = pT; s->pL = pL; s->pB = pB; s->pR = pR; s->dH = dH; s->dW = dW;
    s->OH = ogref_conv_out_size(H, KH, sH, pT, pB, dH);
    s->OW = ogref_conv_out_size(W, KW, sW, pL, pR, dW);
    return s->OH >= 1 && s->OW >= 1;
}

/* One output (n, oc, oy, ox) of the convolution, the definition written out. */
static float conv_one(const struct conv_shape *s, const float *x, const float *w, int64_t n,
                      int64_t oc, int64_t oy, int64_t ox, int mode)
{
    const int64_t cin_g = s->Cin / s->G;
    const int64_t g = oc / (s->Cout / s->G);
    float acc = 0.0f;
    for (int64_t c = 0; c < cin_g; c++)
        for (int64_t ky = 0; ky < s->KH; ky++)
            for (int64_t kx = 0; kx < s->KW; kx++) {
                const int64_t iy = oy * s->sH - s->pT + ky * s->dH;
                const int64_t ix = ox * s->sW - s->pL + kx * s->dW;
                float v = 0.0f;
                if (iy >= 0 && iy < s->H && ix >= 0 && ix < s->W)
                    v = x[((n * s->Cin + g * cin_g + c) * s->H + iy) * s->W + ix];
                const float wt = w[((oc * cin_g + c) * s->KH + ky) * s->KW + kx];
                acc = add_term(acc, wt, v, mode);
            }
    return store_value(acc);
}

int ogref_conv2d_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                        int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                        int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                        int64_t dilH, int64_t dilW, const float *x, const float *w, float *y,
                        int mode)
{
    struct conv_shape s;
    if (!conv_shape_init(&s, N, Cin, H, W, Cout, G, KH, KW, strideH, strideW, padTop, padLeft,
                         padBottom, padRight, dilH, dilW, x, w, y, mode))
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < s.N; n++)
        for (int64_t oc = 0; oc < s.Cout; oc++)
            for (int64_t oy = 0; oy < s.OH; oy++)
                for (int64_t ox = 0; ox < s.OW; ox++)
                    y[((n * s.Cout + oc) * s.OH + oy) * s.OW + ox] =
                        conv_one(&s, x, w, n, oc, oy, ox, mode);
    return 0;
}

int ogref_conv2d_f32_at(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                        int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                        int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                        int64_t dilH, int64_t dilW, const float *x, const float *w,
                        int64_t npts, const int64_t *flat, float *out, int mode)
{
    struct conv_shape s;
    if (!conv_shape_init(&s, N, Cin, H, W, Cout, G, KH, KW, strideH, strideW, padTop, padLeft,
                         padBottom, padRight, dilH, dilW, x, w, out ? out : x, mode) ||
        npts < 0)
        return -1;
    if (npts > 0 && (flat == NULL || out == NULL))
        return -1;
    const int64_t total = s.N * s.Cout * s.OH * s.OW;
    for (int64_t t = 0; t < npts; t++)
        if (flat[t] < 0 || flat[t] >= total)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npts; t++) {
        int64_t r = flat[t];
        const int64_t ox = r % s.OW;
        r /= s.OW;
        const int64_t oy = r % s.OH;
        r /= s.OH;
        const int64_t oc = r % s.Cout;
        const int64_t n = r / s.Cout;
        out[t] = conv_one(&s, x, w, n, oc, oy, ox, mode);
    }
    return 0;
}

int ogref_conv2d_im2col_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                               int64_t G, int64_t KH, int64_t KW, int64_t strideH,
                               int64_t strideW, int64_t padTop, int64_t padLeft,
                               int64_t padBottom, int64_t padRight, int64_t dilH,
                               int64_t dilW, const float *x, const float *w, float *y,
                               int mode)
{
    struct conv_shape s;
    if (!conv_shape_init(&s, N, Cin, H, W, Cout, G, KH, KW, strideH, strideW, padTop, padLeft,
                         padBottom, padRight, dilH, dilW, x, w, y, mode))
        return -1;
    const int64_t cin_g = s.Cin / s.G, cout_g = s.Cout / s.G;
    const int64_t K = cin_g * s.KH * s.KW, npix = s.OH * s.OW;
    float *col = (float *)malloc((size_t)K * (size_t)npix * sizeof(float));
    if (col == NULL)
        return -1;
    for (int64_t n = 0; n < s.N; n++)
        for (int64_t g = 0; g < s.G; g++) {
            /* the im2col matrix of image n, group g: row (c, ky, kx), column (oy, ox) */
#pragma omp parallel for collapse(3) schedule(static)
            for (int64_t c = 0; c < cin_g; c++)
                for (int64_t ky = 0; ky < s.KH; ky++)
                    for (int64_t kx = 0; kx < s.KW; kx++) {
                        const int64_t row = (c * s.KH + ky) * s.KW + kx;
                        for (int64_t oy = 0; oy < s.OH; oy++)
                            for (int64_t ox = 0; ox < s.OW; ox++) {
                                const int64_t iy = oy * s.sH - s.pT + ky * s.dH;
                                const int64_t ix = ox * s.sW - s.pL + kx * s.dW;
                                float v = 0.0f;
                                if (iy >= 0 && iy < s.H && ix >= 0 && ix < s.W)
                                    v = x[((n * s.Cin + g * cin_g + c) * s.H + iy) * s.W + ix];
                                col[row * npix + oy * s.OW + ox] = v;
                            }
                    }
            /* the group's weights [cout_g, K] times the im2col matrix [K, npix]:
             * the product's loop-interchanged form (each output still summed
             * from +0 in increasing k) */
            int rc = ogref_gemm_f32_rowwise(cout_g, npix, K, w + g * cout_g * K, K, col, npix,
                                            y + (n * s.Cout + g * cout_g) * npix, npix, mode);
            if (rc != 0) {
                free(col);
                return rc;
            }
        }
    free(col);
    return 0;
}

int ogref_selftest(void)
{
    /* 1 + 2^-11 and 1 + 2^-12 are exact binary32 values. */
    const float a[2] = {1.0f + 0x1p-11f, -(1.0f + 0x1p-12f)};
    const float b[2] = {1.0f, 1.0f + 0x1p-12f};
    float ce = 1.0f, cf = 1.0f;
    if (ogref_gemm_f32(1, 1, 2, a, 2, b, 1, &ce, 1, MODE_EXACT) != 0)
        return -1;
    if (ogref_gemm_f32(1, 1, 2, a, 2, b, 1, &cf, 1, MODE_FAST) != 0)
        return -1;
    uint32_t ue, uf;
    memcpy(&ue, &ce, 4);
    memcpy(&uf, &cf, 4);
    if (ue != 0x00000000u)
        return -2;
    if (uf != 0xB3800000u)
        return -3;
    return 0;
}

int ogref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int ogref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* The convolution epilogue: bias of the output channel, then the activation,
 * then the residual, after the whole sum ("Convolution (fast mode)", section
 * "Tiles and chunks": bias, then activation; section "Single-column
 * products": the bias, activation and residual epilogue). */
int ogref_conv_epilogue_f32(int64_t N, int64_t Cout, int64_t OHW, float *y, const float *bias,
                            int act, const float *residual)
{
    if (act != 0 && act != 1)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t oc = 0; oc < Cout; ++oc)
            for (int64_t i = 0; i < OHW; ++i) {
                const int64_t at = (n * Cout + oc) * OHW + i;
                float v = y[at];
                if (bias)
                    v = v + bias[oc];
                if (act == 1 && !isnan(v) && !(v > 0.0f))
                    v = 0.0f;
                if (residual)
                    v = v + residual[at];
                y[at] = store_value(v);
            }
    return 0;
}
