// og_kernels.hpp -- device code of libog: the exact and fast fp32 matrix
// product and the implicit-GEMM NCHW convolution for gfx950.
//
// Every output is owned by exactly one lane and receives all of its terms,
// in increasing k, in that lane's registers, starting from +0 ("Exact mode",
// rules 2, 3 and 5; "Matrix product and convolution kernels", section "Fixed
// chunks and thread independence").  A workgroup owns one output tile of one
// group and walks the whole of k; k is never split across lanes, waves or
// workgroups.
//
// Per term the two modes do:
//   exact: prod = round(a*b); acc = round(acc + prod)          ("Exact mode")
//   fast : acc = round(a*b + acc), one fused multiply-add      ("Fast mode")
//
// The matrix-core kernel uses the fp32 MFMA with one k per instruction
// (v_mfma_f32_32x32x1_2b_f32): for every element of its 32x32 blocks it
// computes D = fma(a_i, b_j, C) with a single rounding, subnormals kept
// (checked on gfx950 against a correctly rounded fma on every class of
// input).  A chain of them over increasing k is therefore exactly the fast
// mode's ordered fused multiply-add.  Exact mode takes the rounded product
// from the same instruction with C = +0 (fma(a, b, +0) is round(a*b) except
// that an exact zero product comes out +0 instead of -0, which cannot change
// acc + prod because acc is never -0) and adds it on the VALU with a
// separately rounded v_add_f32.
//
// Operands are staged through LDS in k-chunks of BK: the A tile (weights, or
// the left matrix) and the B tile (the right matrix, or the convolution's
// input patches gathered on the fly with the zero padding written during the
// gather; "Convolution (fast mode)", section "Layout of the work").  Rows,
// columns and taps beyond the problem are staged as +0 in BOTH operands, so
// the extra terms are fma(+0, +0, acc) = acc and acc + round(+0 * +0) = acc.
//
// All code is compiled with -ffp-contract=off and with fp32 denormals on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace og {

typedef float f32x32 __attribute__((ext_vector_type(32)));

enum Mode { kExact = 0, kFast = 1 };

// How the B operand of the implicit product is read.
enum BKind {
  kBMatrix = 0,   // row-major matrix, element (t, j) at B[t*ldb + j]
  kBGather = 1,   // convolution patches, gathered with zero padding
  kBPlanes = 2,   // 1x1 / stride 1 / no padding: input planes read in place
};

// One launch: an implicit matrix product C_g = A_g * B_g for each group g.
// M, N, K are per group.  For a convolution M = Cout/G, K = Cin/G*KH*KW and
// the N columns are the output pixels of all images (n, oy, ox), images
// folded into one column range.
struct Problem {
  const float *A;      // A_g element (i, t) at A[g*a_gstride + i*lda + t]
  int64_t lda, a_gstride;
  const float *B;      // matrix: element (t, j) at B[t*ldb + j]; conv: the input x
  int64_t ldb;
  float *C;            // matrix: C[i*ldc + j]; conv: the output y
  int64_t ldc;
  int M, N, K, groups;
  int tiles_m, tiles_n;
  // convolution only
  int H, W, OW, OHW, KW, KHW, sH, sW, pT, pL, dH, dW;
  int64_t x_img, x_grp;  // element strides of x between images and between groups
  int64_t y_img, y_grp;  // element strides of y between images and between groups
};

// ---------------------------------------------------------------------------
// Workgroup -> tile.  Workgroups are handed to the 8 XCDs of the chip in
// turn (workgroup b runs on XCD b mod 8).  The remap gives every XCD one
// contiguous range of tiles, and within a group the tiles run in bands of
// kBand tile-rows, column by column, so the tiles that run at the same time
// on one XCD share A rows and B columns in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kBand = 8;

struct TileCoord {
  int g, tm, tn;
};

__host__ __device__ inline TileCoord tile_of_block(int bid, int nblocks, int tiles_m,
                                                   int tiles_n) {
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  const int t = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int per_group = tiles_m * tiles_n;
  TileCoord c;
  c.g = t / per_group;
  const int r = t - c.g * per_group;
  const int band = r / (kBand * tiles_n);
  const int rows = min(kBand, tiles_m - band * kBand);
  const int idx = r - band * kBand * tiles_n;
  c.tm = band * kBand + idx % rows;
  c.tn = idx / rows;
  return c;
}

__device__ inline float canonical(float v) {
  return v != v ? __uint_as_float(0x7FC00000u) : v;
}

// ---------------------------------------------------------------------------
// Staging of one k-chunk.  A: thread -> (row r0 + q*rstep, tap c); coalesced
// along k.  B: thread -> (column, taps kk0 + q*kstep); coalesced along the
// columns.  Values go to registers first, then to the LDS buffer not being
// read, so the global loads of chunk c+1 overlap the products of chunk c.
// ---------------------------------------------------------------------------
template <int BM, int BK, int NT>
struct ALoader {
  static constexpr int kPer = BM * BK / NT;
  static constexpr int kRstep = NT / BK;
  const float *ptr;  // row r0, tap c of chunk 0
  int64_t row_step;  // kRstep rows
  int c, r0, rows_left;

  __device__ void init(const Problem &p, int g, int m0, int tid) {
    c = tid % BK;
    r0 = tid / BK;
    rows_left = p.M - m0 - r0;  // row q is valid when q*kRstep < rows_left
    ptr = p.A + g * p.a_gstride + (int64_t)(m0 + r0) * p.lda + c;
    row_step = (int64_t)kRstep * p.lda;
  }
  __device__ void load(const Problem &p, int k0, float (&r)[kPer]) const {
    const bool kin = k0 + c < p.K;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const bool ok = kin && q * kRstep < rows_left;
      const float v = *(ok ? ptr + q * row_step + k0 : p.A);  // p.A: any readable element
      r[q] = ok ? v : 0.0f;
    }
  }
  template <int LDA_STRIDE>
  __device__ void store(float *lds, const float (&r)[kPer]) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) lds[c * LDA_STRIDE + r0 + q * kRstep] = r[q];
  }
};

template <int BN, int BK, int NT, int KIND>
struct BLoader {
  static constexpr int kPer = BN * BK / NT;
  static constexpr int kKstep = NT / BN;
  int col, kk0;
  bool col_ok;
  int64_t base;  // per-thread element offset of the column's data
  int iy0, ix0;  // gather: top-left input position of the column's window

  __device__ void init(const Problem &p, int g, int n0, int tid) {
    col = tid % BN;
    kk0 = __builtin_amdgcn_readfirstlane(tid / BN);  // uniform in a wave (BN >= 64)
    const int j = n0 + col;
    col_ok = j < p.N;
    if (KIND == kBMatrix) {
      base = j;
    } else {
      const int jj = col_ok ? j : 0;
      const int img = jj / p.OHW;
      const int pix = jj - img * p.OHW;
      if (KIND == kBPlanes) {
        base = img * p.x_img + g * p.x_grp + pix;
      } else {
        const int oy = pix / p.OW;
        const int ox = pix - oy * p.OW;
        iy0 = oy * p.sH - p.pT;
        ix0 = ox * p.sW - p.pL;
        base = img * p.x_img + g * p.x_grp + (int64_t)iy0 * p.W + ix0;
      }
    }
  }
  __device__ void load(const Problem &p, int k0, float (&r)[kPer]) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int t = k0 + kk0 + q * kKstep;  // wave-uniform tap index
      // The load always runs, from p.B (any readable element) when the
      // element is outside the problem, and its value is then replaced by +0.
      bool ok = col_ok && t < p.K;
      int64_t off = 0;
      if (KIND == kBMatrix) {
        off = base + (int64_t)t * p.ldb;
      } else if (KIND == kBPlanes) {
        off = base + (int64_t)t * p.OHW;  // plane t of the group
      } else {
        // tap t -> (c, ky, kx): channel, kernel row, kernel column
        const int c = t / p.KHW;
        const int rr = t - c * p.KHW;
        const int ky = rr / p.KW;
        const int kx = rr - ky * p.KW;
        const int dy = ky * p.dH, dx = kx * p.dW;
        const bool inside = (unsigned)(iy0 + dy) < (unsigned)p.H &&
                            (unsigned)(ix0 + dx) < (unsigned)p.W;
        ok = ok && inside;  // outside the plane: a padding tap, +0
        off = base + (int64_t)c * p.H * p.W + (int64_t)dy * p.W + dx;
      }
      const float v = p.B[ok ? off : 0];
      r[q] = ok ? v : 0.0f;
    }
  }
  __device__ void store(float *lds, const float (&r)[kPer]) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) lds[(kk0 + q * kKstep) * BN + col] = r[q];
  }
};

// Pointer to output (row, col) of group g, or nullptr outside the problem.
template <int KIND>
__device__ inline float *out_ptr(const Problem &p, int g, int row, int col) {
  if (KIND == kBMatrix) return p.C + (int64_t)row * p.ldc + col;
  const int img = col / p.OHW;
  const int pix = col - img * p.OHW;
  return p.C + img * p.y_img + g * p.y_grp + (int64_t)row * p.OHW + pix;
}

// ---------------------------------------------------------------------------
// Matrix-core kernel.  256 threads = 4 waves arranged WM x WN; a wave owns a
// (TM*32) x (TN*64) sub-tile as TM x TN blocks of 32 x 64 outputs, each block
// one 32x32x1 MFMA pair-of-blocks: lanes 0-31 and 32-63 both carry the 32 A
// rows, lanes 0-31 carry B columns 0-31 and lanes 32-63 columns 32-63.
// ---------------------------------------------------------------------------
template <int MODE, int BM, int BN, int WM, int WN, int KIND>
__global__ void __launch_bounds__(256) mfma_kernel(Problem p) {
  constexpr int NT = 256, BK = 16;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 64;
  static_assert(WM * WN == 4 && TM >= 1 && TN >= 1, "tile shape");
  constexpr int LDA = BM + 1;  // k-major A tile, padded against bank conflicts of the transposing store
  __shared__ __align__(16) float As[2][BK * LDA];
  __shared__ __align__(16) float Bs[2][BK * BN];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  ALoader<BM, BK, NT> al;
  BLoader<BN, BK, NT, KIND> bl;
  al.init(p, tc.g, m0, tid);
  bl.init(p, tc.g, n0, tid);
  float ra[ALoader<BM, BK, NT>::kPer];
  float rb[BLoader<BN, BK, NT, KIND>::kPer];

  f32x32 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x32{};

  const int nchunks = (p.K + BK - 1) / BK;
  if (nchunks > 0) {
    al.load(p, 0, ra);
    bl.load(p, 0, rb);
    al.template store<LDA>(As[0], ra);
    bl.store(Bs[0], rb);
  }
  __syncthreads();

  const int a_off = wm * TM * 32 + (lane & 31);
  const int b_off = wn * TN * 64 + lane;
  for (int kc = 0; kc < nchunks; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nchunks;
    if (more) {
      al.load(p, (kc + 1) * BK, ra);
      bl.load(p, (kc + 1) * BK, rb);
    }
    const float *as = As[cur];
    const float *bs = Bs[cur];
    if (MODE == kFast) {
      float a[2][TM], b[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[0][i] = as[a_off + i * 32];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[0][j] = bs[b_off + j * 64];
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        const int u = kk & 1;
        if (kk + 1 < BK) {  // operands of the next k, read while this k's MFMAs run
#pragma unroll
          for (int i = 0; i < TM; ++i) a[u ^ 1][i] = as[(kk + 1) * LDA + a_off + i * 32];
#pragma unroll
          for (int j = 0; j < TN; ++j) b[u ^ 1][j] = bs[(kk + 1) * BN + b_off + j * 64];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
      }
    } else {
      // Exact: the rolled k loop keeps the products of one k live at a time
      // (an unrolled loop lets the compiler make every product of the chunk
      // first); waves sharing a SIMD overlap one another's MFMAs and adds.
#pragma unroll 1
      for (int kk = 0; kk < BK; ++kk) {
        float a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = as[kk * LDA + a_off + i * 32];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = bs[kk * BN + b_off + j * 64];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const f32x32 prod = __builtin_amdgcn_mfma_f32_32x32x1f32(a[i], b[j], f32x32{}, 0, 0, 0);
            acc[i][j] += prod;
          }
      }
    }
    if (more) {
      al.template store<LDA>(As[cur ^ 1], ra);
      bl.store(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }

  // Epilogue: accumulator register r of lane l in block pair half h = r/16
  // holds row 8*((r%16)/4) + 4*(l/32) + r%4 and column h*32 + l%32 of the
  // 32 x 64 block.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = n0 + wn * TN * 64 + j * 64 + h * 32 + (lane & 31);
        if (col >= p.N) continue;
        float *base = out_ptr<KIND>(p, tc.g, 0, col);
        const int64_t rstride = KIND == kBMatrix ? p.ldc : (int64_t)p.OHW;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * TM * 32 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M) base[row * rstride] = canonical(acc[i][j][h * 16 + r]);
        }
      }
}

// ---------------------------------------------------------------------------
// VALU kernel: 64 x 64 tile, 256 threads in a 16 x 16 grid, each thread a
// 4 x 4 micro-tile (rows ty*4.., columns tx*4..).  Per term: v_fma_f32 in fast
// mode, v_mul_f32 then v_add_f32 in exact mode.
// ---------------------------------------------------------------------------
template <int MODE, int KIND>
__global__ void __launch_bounds__(256) valu_kernel(Problem p) {
  constexpr int NT = 256, BK = 16, BM = 64, BN = 64;
  constexpr int LDA = BM + 4;
  __shared__ __align__(16) float As[2][BK * LDA];
  __shared__ __align__(16) float Bs[2][BK * BN];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  ALoader<BM, BK, NT> al;
  BLoader<BN, BK, NT, KIND> bl;
  al.init(p, tc.g, m0, tid);
  bl.init(p, tc.g, n0, tid);
  float ra[ALoader<BM, BK, NT>::kPer];
  float rb[BLoader<BN, BK, NT, KIND>::kPer];

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  const int nchunks = (p.K + BK - 1) / BK;
  if (nchunks > 0) {
    al.load(p, 0, ra);
    bl.load(p, 0, rb);
    al.template store<LDA>(As[0], ra);
    bl.store(Bs[0], rb);
  }
  __syncthreads();
  for (int kc = 0; kc < nchunks; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nchunks;
    if (more) {
      al.load(p, (kc + 1) * BK, ra);
      bl.load(p, (kc + 1) * BK, rb);
    }
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4 *>(&As[cur][kk * LDA + ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4 *>(&Bs[cur][kk * BN + tx * 4]);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
      const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (MODE == kFast) {
            acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
          } else {
            const float prod = a[i] * b[j];
            acc[i][j] = acc[i][j] + prod;
          }
        }
    }
    if (more) {
      al.template store<LDA>(As[cur ^ 1], ra);
      bl.store(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + tx * 4 + j;
    if (col >= p.N) continue;
    float *base = out_ptr<KIND>(p, tc.g, 0, col);
    const int64_t rstride = KIND == kBMatrix ? p.ldc : (int64_t)p.OHW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      if (row < p.M) base[row * rstride] = canonical(acc[i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Lane kernel, for shapes with few outputs and long k (the deep layers of a
// convolution network at batch 1, short matrix products): the matrix-core
// instructions take 64 (32x32x1) or ~13 (4x4x1) cycles per dependent k step,
// a VALU fused multiply-add about 5.  Lane l of a wave owns output column
// n0 + l for the wave's R output rows; the R weights of a k step are the
// same for every lane and come through the scalar cache into SGPRs; the B
// value of the step is read from the LDS tile all W waves of the block
// share (staged like the matrix-core kernel's, zero padding included).
// ---------------------------------------------------------------------------
template <int MODE, int KIND, int R, int W>
__global__ void __launch_bounds__(64 * W) lane_kernel(Problem p, const float *__restrict__ Aw) {
  constexpr int NT = 64 * W, BK = 32, BN = 64;
  __shared__ __align__(16) float Bs[2][BK * BN];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = tc.tn * BN;
  const int row0 = tc.tm * (R * W) + wave * R;

  BLoader<BN, BK, NT, KIND> bl;
  bl.init(p, tc.g, n0, tid);
  float rb[BLoader<BN, BK, NT, KIND>::kPer];

  // Weight rows of this wave; a row beyond M reads row M-1 and is never stored.
  const float *arow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.M - 1);
    arow[r] = Aw + tc.g * p.a_gstride + (int64_t)row * p.lda;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  const int nchunks = (p.K + BK - 1) / BK;
  if (nchunks > 0) {
    bl.load(p, 0, rb);
    bl.store(Bs[0], rb);
  }
  __syncthreads();
  for (int kc = 0; kc < nchunks; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nchunks;
    if (more) bl.load(p, (kc + 1) * BK, rb);
    const int k0 = kc * BK;
    const float *bs = Bs[cur];
    if (k0 + BK <= p.K) {
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        const float b = bs[kk * BN + lane];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float a = arow[r][k0 + kk];
          if (MODE == kFast) {
            acc[r] = __builtin_fmaf(a, b, acc[r]);
          } else {
            const float prod = a * b;
            acc[r] = acc[r] + prod;
          }
        }
      }
    } else {
      // last, partial chunk: taps at or beyond K are +0 in both operands
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        const float b = bs[kk * BN + lane];
        const bool kin = k0 + kk < p.K;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float av = arow[r][kin ? k0 + kk : 0];
          const float a = kin ? av : 0.0f;
          if (MODE == kFast) {
            acc[r] = __builtin_fmaf(a, b, acc[r]);
          } else {
            const float prod = a * b;
            acc[r] = acc[r] + prod;
          }
        }
      }
    }
    if (more) bl.store(Bs[cur ^ 1], rb);
    __syncthreads();
  }
  const int col = n0 + lane;
  if (col < p.N) {
    float *base = out_ptr<KIND>(p, tc.g, 0, col);
    const int64_t rstride = KIND == kBMatrix ? p.ldc : (int64_t)p.OHW;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row0 + r < p.M) base[(row0 + r) * rstride] = canonical(acc[r]);
  }
}

}  // namespace og
