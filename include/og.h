/*
 * og.h -- exact and fast fp32 matrix product and NCHW convolution on AMD
 * Instinct MI355X (gfx950).  C ABI of libog.so.
 *
 * What the library computes is defined by two pages of the OneModel
 * documentation:
 *  - "Exact mode", sections "Rules every exact kernel follows", "Matrix
 *    product" and "Convolution": every output is one accumulator that starts
 *    at +0 and receives its terms in increasing index (for a convolution:
 *    channel, then kernel row, then kernel column), each product and each sum
 *    rounded to binary32 on its own (round to nearest even, subnormals kept);
 *    a NaN result is stored as 0x7FC00000; an empty sum is +0; no bias.
 *  - "Matrix product and convolution kernels", section "Fast mode", and
 *    "Convolution (fast mode)", section "What each output is": the same
 *    accumulator and order with one fused multiply-add per term.  This
 *    library also stores a NaN result of fast mode as 0x7FC00000, so both
 *    modes have exactly one correct bit pattern per output.
 * In exact and fast mode results do not depend on tile shapes, kernel
 * variant, stream or device: every output is computed whole by one GPU lane
 * over all of k, and k is never split ("Matrix product and convolution
 * kernels", section "Fixed chunks and thread independence").  A third mode,
 * OG_MODE_FAST_MFMA, trades that order for a stated error bound (below).
 *
 * Conventions of every entry point below:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library allocates nothing, keeps no pointer after it returns and frees
 *    nothing.  Outputs must not overlap inputs.
 *  - Work is queued on the calling thread's current stream (og_set_stream)
 *    and the call returns without waiting for it.  Argument errors are
 *    returned before anything is queued; a fault inside a kernel surfaces at
 *    the caller's next synchronisation.
 *  - On an error nothing is written, and og_last_error() describes it.
 *  - Only gfx950 is supported: on any other device a compute call returns
 *    OG_ERR_DEVICE (there is no fallback path).
 */
#ifndef OG_H
#define OG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int og_status;

#define OG_OK 0
#define OG_ERR_INVALID_ARG (-1) /* a size, stride, pointer or mode is out of range           */
#define OG_ERR_NOT_EXACT (-2)   /* exact or fast mode asked of a kernel variant that cannot
                                   give that mode's bits (the split-k variants 21..25):
                                   reported, never approximated ("Exact mode")             */
#define OG_ERR_DEVICE (-3)      /* HIP error, or the current device is not gfx950            */
#define OG_ERR_TOO_LARGE (-4)   /* a dimension does not fit the kernels' 32-bit offsets and
                                   counters: m, n or k above 2^31-1, lda or ldb above 2^22, a
                                   convolution's Cin/G*KH*KW above 2^22 or input above 2^29
                                   elements (each entry point states its bounds)           */

#define OG_MODE_EXACT 0 /* separately rounded multiply and add ("Exact mode")              */
#define OG_MODE_FAST 1  /* one fused multiply-add per term, same order ("Fast mode")        */
/*
 * OG_MODE_FAST_MFMA: fast mode under a stated tolerance instead of an order.
 * Every output is the sum over all of k of its products, but the terms may
 * be grouped and added in any order: k is split among the waves of a
 * workgroup (never among workgroups) and summed four products at a time by
 * the fp32 matrix-core instruction v_mfma_f32_16x16x4_f32, whose internal
 * order is not specified.  For each output with exact sum r (real
 * arithmetic), S = sum over p of |a_p * b_p| and K terms, a finite result c
 * satisfies |c - r| <= 4e-6 * sqrt(K) * S + 1e-30 (the accuracy bound of
 * "Matrix product and convolution kernels", section "Fast mode", k*u*S plus
 * 1e-30 for subnormals, in the 4e-6*sqrt(K) form of the dotLLM pull request
 * "F32 outer-product tiled GEMM kernel for prefill", section "Tests"); a
 * result is NaN (stored as 0x7FC00000) or an infinity of the exact result's
 * sign exactly when the exact result is.  Results repeat bit for bit from run
 * to run and do not depend on the stream, but may change with the kernel
 * variant.  Where the split-k kernels are not expected to be faster the
 * fast-mode kernels run (they meet the bound).
 */
#define OG_MODE_FAST_MFMA 2

#define OG_ACT_NONE 0 /* og_conv2d_f32_epi: no activation                                 */
#define OG_ACT_RELU 1 /* og_conv2d_f32_epi: v > 0 ? v : +0 (a NaN stays NaN)              */

/*
 * Matrix product, row-major ("Matrix product and convolution kernels",
 * first paragraph; "Exact mode", section "Matrix product"):
 *
 *     C[i*ldc + j] = sum over p = 0..k-1 of A[i*lda + p] * B[p*ldb + j]
 *
 * for 0 <= i < m, 0 <= j < n, summed by the mode's rule.  C is overwritten
 * (there is no alpha, beta or bias); the gaps C[i*ldc + j], n <= j < ldc, are
 * never written.  Requirements: m, n, k >= 0; lda >= max(1,k),
 * ldb >= max(1,n), ldc >= max(1,n); A and B non-null when m, n and k are all
 * positive, C non-null when m and n are positive.  m == 0 or n == 0: nothing
 * is done.  k == 0: every output is +0 and A, B are not read.
 * OG_ERR_TOO_LARGE when m, n or k exceeds 2^31-1 or lda or ldb exceeds 2^22.
 */
og_status og_gemm_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, int mode);

/*
 * Matrix product with the right operand given as its transpose: B is n x k,
 * row-major, so that each of its rows holds the k weights of one output
 * column (the weights-as-N-x-K layout of the dotLLM pull request "F32
 * outer-product tiled GEMM kernel for prefill", section "Kernel design"):
 *
 *     C[i*ldc + j] = sum over p = 0..k-1 of A[i*lda + p] * B[j*ldb + p]
 *
 * that is, C = A * B^T, each output summed by the mode's rule in increasing p
 * from +0 ("Exact mode", section "Matrix product": the product of two
 * elements commutes, so this is the matrix product of A and B^T, bit for
 * bit).  Same contract as og_gemm_f32 except that ldb >= max(1,k).  With
 * m == 1 it is a single-row product against the rows of B, streamed once
 * ("Convolution (fast mode)", section "Single-column products").  Every
 * kernel variant 1..5, 17 and 20 has a form for it; other variants run as 0.
 */
og_status og_gemm_nt_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                         const float *B, int64_t ldb, float *C, int64_t ldc, int mode);

/*
 * 2-D convolution, NCHW, per-axis stride, padding and dilation ("Exact mode",
 * section "Convolution"; "Convolution (fast mode)", sections "What each output
 * is" and "Layout of the work"):
 *
 *   x [N, Cin, H, W], w [Cout, Cin/G, KH, KW], y [N, Cout, OH, OW], contiguous;
 *   output (n, oc, oy, ox) of group g = oc / (Cout/G) sums, over c in
 *   [0, Cin/G), then ky in [0, KH), then kx in [0, KW), the products
 *   w[oc][c][ky][kx] * v, where v is x[n][g*Cin/G + c][iy][ix] with
 *   iy = oy*strideH - padTop + ky*dilH and ix = ox*strideW - padLeft + kx*dilW
 *   when 0 <= iy < H and 0 <= ix < W, and +0 otherwise.  Taps in the padding
 *   are real products with +0 (an infinite or NaN weight there gives NaN).
 *   OH and OW follow og_conv2d_out_size.  No bias.
 *
 * It runs as an implicit matrix product per group: the weights are A and the
 * input patches are gathered into on-chip tiles of B, the zero padding written
 * during the gather and never stored in memory.  A one-dimensional
 * convolution is H = 1, KH = 1 with padTop = padBottom = 0.
 * Requirements: N, Cin, H, W, Cout, G, KH, KW >= 1; strides and dilations
 * >= 1; pads >= 0; Cin and Cout multiples of G; OH, OW >= 1; pointers
 * non-null.  OG_ERR_TOO_LARGE when the input holds more than 2^29 elements,
 * when K = Cin/G*KH*KW (the taps of one output, the row stride of the
 * weights) exceeds 2^22, or when a size does not fit 31 bits (the kernels
 * form 32-bit offsets).
 */
og_status og_conv2d_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                           int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                           int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                           int64_t dilH, int64_t dilW, const float *x, const float *w, float *y,
                           int mode);

/*
 * og_conv2d_f32_ex followed by the convolution epilogue ("Convolution (fast
 * mode)", section "Tiles and chunks": bias, then activation, applied to each
 * finished output with rows counted from the group's first output channel;
 * section "Single-column products": the bias, activation and residual
 * epilogue).  For output (n, oc, oy, ox) with sum s (summed by the mode's
 * rule, exactly as og_conv2d_f32_ex does):
 *
 *     v = s + bias[oc]                       (if bias is not NULL; rounded)
 *     v = v > 0 ? v : +0, NaN kept           (if act == OG_ACT_RELU)
 *     v = v + residual[n][oc][oy][ox]        (if residual is not NULL; rounded)
 *     y[n][oc][oy][ox] = isNaN(v) ? 0x7FC00000 : v
 *
 * bias: Cout floats; residual: a contiguous [N, Cout, OutH, OutW] tensor
 * (it may be y itself: each output reads its own residual before writing);
 * both device pointers owned by the caller, NULL for none.  act must be
 * OG_ACT_NONE or OG_ACT_RELU, else OG_ERR_INVALID_ARG; otherwise the contract
 * of og_conv2d_f32_ex.  With no bias, no activation and no residual the
 * result equals og_conv2d_f32_ex's.
 */
og_status og_conv2d_f32_epi(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                            int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                            int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                            int64_t dilH, int64_t dilW, const float *x, const float *w,
                            const float *bias, int act, const float *residual, float *y,
                            int mode);

/*
 * The same convolution with one stride, one symmetric padding and one
 * dilation for both axes: og_conv2d_f32_ex(..., stride, stride, pad, pad,
 * pad, pad, dil, dil, ...).
 */
og_status og_conv2d_f32(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t G,
                        int64_t KH, int64_t KW, int64_t stride, int64_t pad, int64_t dil,
                        const float *x, const float *w, float *y, int mode);

/*
 * Output length of one axis ("Exact mode", section "Convolution"):
 * floor((size + padBefore + padAfter - dil*(k-1) - 1) / stride) + 1.
 * Returns a value < 1 when the window does not fit or an argument is out of
 * range (size, k, stride, dil < 1 or a pad < 0).  Host-only, no device use.
 */
int64_t og_conv2d_out_size(int64_t size, int64_t k, int64_t stride, int64_t padBefore,
                           int64_t padAfter, int64_t dil);

/*
 * Stream for the calling thread's later calls (a hipStream_t; NULL = the
 * default stream).  The library does not take ownership.  Always OG_OK.
 */
og_status og_set_stream(void *hip_stream);
void *og_get_stream(void);

/*
 * Kernel variant for the calling thread's later calls, for tests that check
 * that the results do not depend on it ("Exact mode", rule 5): 0 = chosen
 * from the shape (the default); 1 = the VALU tile kernel (64x64 tiles);
 * 2, 3, 4, 5 = the matrix-core kernel with 128x256, 128x128, 64x128 and
 * 32x256 output tiles (exact mode runs variants 2, 3 and 17 with 64x128
 * tiles, or 128x128 tiles for a gathered convolution);
 * 6, 7, 8, 9 = the lane kernel (one output column per lane) with 1, 2, 4, 8
 * output rows per wave; 10, 11, 12, 13 = the chain kernel (compute waves
 * that only run the k chain, producer waves that stage B) with 64 columns
 * and 4 rows, 64 columns and 2 rows, 16 columns and 4 rows (a 3x3
 * convolution: 32 columns and 2 rows), 64 columns and 4 rows as two rows
 * per lane; 14, 15, 16 = the chain kernel whose compute waves run the k
 * chain on the matrix cores (v_mfma_f32_4x4x1_16b_f32, 4 rows x 64
 * columns per chain) with 4 waves of 4 rows, 2 waves of 2 x 4 rows and
 * 2 waves of 4 rows (exact mode runs them as 10, 13 and 11); 17 = the
 * matrix-core kernel with 256x256 output tiles and 8 waves (exact mode runs
 * it like variants 2 and 3); 18 = the depthwise kernel (a convolution with
 * Cin/G = 1, any channel multiplier Cout/G: each output's KH*KW terms run
 * directly, one output per lane; "Matrix product and convolution kernels",
 * section "Convolution"), which is also what 0 picks for such a shape;
 * 19 = the grouped direct kernel (a grouped 3x3 convolution with
 * 2 <= Cin/G <= 64 and Cout/G <= 8: one output pixel per lane with all of
 * its group's output channels), also what 0 picks for such a shape;
 * 20 = the matrix-core kernel with 64x64 tiles of four waves of 16x64
 * outputs (v_mfma_f32_16x16x1_4b_f32).
 * 21..25 = the split-k kernels of OG_MODE_FAST_MFMA, output tiles of
 * (rows x columns, waves sharing k) = (16 x 16, 16), (16 x 32, 8),
 * (32 x 32, 8), (32 x 64, 4) and (32 x 32, 4); a compute call in exact or
 * fast mode with one of them forced returns OG_ERR_NOT_EXACT (neither
 * mode's bits can come from them).  In OG_MODE_FAST_MFMA a forced variant
 * 1..20 runs that fast-mode kernel.
 * 26, 27, 28 = the halo kernel (3x3 convolutions with horizontal dilation
 * 1): 64 output pixels of one image per block, the input rows their
 * windows reach staged in LDS with the padding in place, each 4 output
 * channels on the matrix cores (v_mfma_f32_4x4x1_16b_f32 with the weights
 * broadcast from one block; fast mode: the k chain itself, exact mode: the
 * rounded products, summed by separately rounded adds in k order); 4
 * waves of 4 rows, 4 waves of 2 x 4 rows and 8 waves of 4 rows.  On shapes
 * they do not take (or whose block does not fit the LDS) they run as 0
 * does.
 * 29, 30 = the panel kernel (fast mode, og_gemm_f32 products and 1x1
 * convolutions): panels of 64 columns of B (input pixels) loaded straight
 * into LDS stages, the weight rows of each wave through its own LDS
 * stages, the k chain of each 4 rows on the matrix cores as in 26..28;
 * 4 waves of 4 rows and 4 waves of 2 x 4 rows.  In exact mode, and on
 * shapes they do not take (other windows), they run as 0 does.
 * 31, 32, 33 = the halo kernel with DPP steps in place of the matrix
 * cores (for latency-bound 3x3 convolutions, a small batch): a lane's own
 * output channels, each step one v_fmac_f32 (exact: v_mul_f32 then a
 * separately rounded add) with the weight broadcast within rows of 16
 * lanes; 4 waves of 1 row, 8 waves of 1 row and 4 waves of 2 rows.  On
 * shapes they do not take they run as 0 does.
 * Every variant runs every shape (a convolution window other than 1x1 or
 * 3x3 runs variants 10..16 as variant 6; variants 18 and 19 run shapes
 * outside their own, and any matrix product, as 0 does).  A value outside
 * 0..33 returns OG_ERR_INVALID_ARG.
 */
og_status og_set_variant(int variant);
int og_get_variant(void);

/*
 * The kernel variant (numbered as for og_set_variant) that og_gemm_f32
 * runs under the automatic choice (variant 0) for an m x n x k product with
 * n >= 2 in `mode`: a tile variant (2..17 or 20), a panel variant (29, 30;
 * fast mode) or a split-k variant (21..25; OG_MODE_FAST_MFMA).  The choice
 * depends on the shape and mode alone, never on the data or the device
 * ("Matrix product and convolution kernels", section "Fixed chunks and
 * thread independence"), so callers that report which kernel ran
 * (benchmarks) and tests of the choice can ask for it; exact mode runs
 * variants 2, 3 and 17 on the 64x128 tile (see og_set_variant).  Queues
 * nothing and needs no device.  Returns OG_ERR_INVALID_ARG for a mode
 * other than 0, 1 or 2 or for m < 1, n < 2 or k < 1 (a single column takes
 * the row-dot or streamed-column form, which has no number), and
 * OG_ERR_TOO_LARGE for a dimension above 2^31-1.
 */
int og_gemm_choice(int64_t m, int64_t n, int64_t k, int mode);

/* Description of the calling thread's last error ("" after a success). */
const char *og_last_error(void);

/* Library version, "major.minor.patch". */
const char *og_version(void);

#ifdef __cplusplus
}
#endif
#endif
