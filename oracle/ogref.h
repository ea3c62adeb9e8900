/*
 * ogref.h -- the CPU oracle for the fp32 matrix product and the NCHW convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two never include or
 * import one another.
 *
 * Every routine works on HOST pointers, writes only the outputs it names and
 * returns 0 on success or -1 on an invalid argument (nothing is written then).
 *
 * mode 0 = exact (OneModel "Exact mode": binary32 round-to-nearest-even, the
 *          product and the sum rounded separately, one accumulator per output
 *          starting at +0, terms in increasing index, NaN stored as 0x7FC00000).
 * mode 1 = fast  (OneModel "Matrix product and convolution kernels", section
 *          "Fast mode": one fused multiply-add per term in the same order; the
 *          NaN payload is left open there and is made canonical here too).
 */
#ifndef OGREF_H
#define OGREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* C[i*ldc+j] = sum_p A[i*lda+p]*B[p*ldb+j], one output at a time (the literal
 * per-output loop of the exact-mode page, "Matrix product").  Row-major,
 * lda >= max(1,k), ldb >= max(1,n), ldc >= max(1,n).  k = 0 stores +0. */
int ogref_gemm_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float *C, int64_t ldc, int mode);

/* Same result by the loop interchange i, p, j: each output still receives its
 * terms in increasing p from +0, so the bits are those of ogref_gemm_f32. */
int ogref_gemm_f32_rowwise(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                           const float *B, int64_t ldb, float *C, int64_t ldc, int mode);

/* npts single outputs (rows[t], cols[t]) of the product, written to out[t]. */
int ogref_gemm_f32_at(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                      const float *B, int64_t ldb, int64_t npts, const int64_t *rows,
                      const int64_t *cols, float *out, int mode);

/* Output length of one axis (exact-mode page, "Convolution"):
 * floor((size + padBefore + padAfter - dil*(K-1) - 1) / stride) + 1.
 * Returns a value < 1 when the window does not fit. */
int64_t ogref_conv_out_size(int64_t size, int64_t k, int64_t stride, int64_t pad_before,
                            int64_t pad_after, int64_t dil);

/* Direct convolution, NCHW.  x [N,Cin,H,W], w [Cout,Cin/G,KH,KW],
 * y [N,Cout,OH,OW], all contiguous.  Per output: taps in the order channel,
 * kernel row, kernel column; taps outside the plane read +0 and are still
 * multiplied.  No bias. */
int ogref_conv2d_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                        int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                        int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                        int64_t dilH, int64_t dilW, const float *x, const float *w, float *y,
                        int mode);

/* Same convolution through a materialised im2col matrix per image and group
 * (rows ordered channel, kernel row, kernel column) and ogref_gemm_f32. */
int ogref_conv2d_im2col_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                               int64_t G, int64_t KH, int64_t KW, int64_t strideH,
                               int64_t strideW, int64_t padTop, int64_t padLeft,
                               int64_t padBottom, int64_t padRight, int64_t dilH,
                               int64_t dilW, const float *x, const float *w, float *y,
                               int mode);

/* npts single outputs of the direct convolution, given as flat indices into
 * y [N,Cout,OH,OW], written to out[t]. */
int ogref_conv2d_f32_at(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                        int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                        int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                        int64_t dilH, int64_t dilW, const float *x, const float *w,
                        int64_t npts, const int64_t *flat, float *out, int mode);

/* The convolution epilogue, in place on y [N, Cout, OHW] ("Convolution (fast
 * mode)", sections "Tiles and chunks" and "Single-column products"): per
 * output, v = y + bias[oc] (if bias), then ReLU (act 1: v > 0 ? v : +0, a NaN
 * kept), then v + residual (if residual, same position), each operation
 * rounded on its own, then NaN made canonical.  Returns 0, or -1 for an
 * activation other than 0 or 1. */
int ogref_conv_epilogue_f32(int64_t N, int64_t Cout, int64_t OHW, float *y, const float *bias,
                            int act, const float *residual);

/* Load-time check that the compiled library separates fused from unfused
 * arithmetic:
 * the two-term sum [1+2^-11, -(1+2^-12)] . [1, 1+2^-12] is +0 exactly and
 * -2^-24 fused.  Returns 0 when both hold. */
int ogref_selftest(void);

/* Threads an OpenMP region of this library uses. */
int ogref_num_threads(void);

/* Sets the threads of the library's later OpenMP regions in the calling
 * thread (n >= 1; other values change nothing) and returns the new count.
 * The split is over outputs only, so results do not depend on it. */
int ogref_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
