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
// Operands are staged through LDS in k-chunks: the A tile (weights, or the
// left matrix) and the B tile (the right matrix, or the convolution's input
// patches gathered on the fly with the zero padding written during the
// gather; "Convolution (fast mode)", section "Layout of the work").  The
// global loads of a chunk are issued D-1 chunks ahead into a ring of
// registers, so their latency hides behind the products of the chunks in
// between.  Rows and columns beyond the problem are staged as +0.  Taps
// beyond k (the last chunk running past the end) read +0 in both operands;
// in fast mode one operand's padding then gets its sign bit set (an OR with
// a mask that is zero for real taps, applied only in the chunk that runs
// past k, a uniform test), so each such term adds a product of -0, and
// x + (-0) = x for every x.  A +0 product would not do:
// in fast mode a sum can be -0 (a fused multiply-add whose exact result is a
// negative number too small to represent, added to +0, rounds to -0), and
// -0 + (+0) = +0.  In exact mode a sum is never -0 (+0 + (-0) = +0, and a
// rounded sum of non-zero values is never -0), so +0 padding is neutral.
//
// All code is compiled with -ffp-contract=off and with fp32 denormals on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace og {

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Mode { kExact = 0, kFast = 1 };

// How the B operand of the implicit product is read.
enum BKind {
  kBMatrix = 0,   // row-major matrix, element (t, j) at B[t*ldb + j]
  kBGather = 1,   // convolution patches, gathered with zero padding
  kBPlanes = 2,   // 1x1 / stride 1 / no padding: input planes read in place
  kBMatrixT = 3,  // B given as its transpose, N x K row-major: element (t, j) at B[j*ldb + t]
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
  int H, W, HW, OW, OHW, KH, KW, KHW, sH, sW, pT, pL, pR, dH, dW;  // pR: right pad
  int64_t x_img, x_grp;  // element strides of x between images and between groups
  int64_t y_img, y_grp;  // element strides of y between images and between groups
  int a_vec;             // A rows 16-byte aligned (A, lda and K multiples of 4 floats)
  int bh, ih, iw;        // depthwise band kernel: output rows per band, staged input rows, columns
  int hrows;             // halo kernel: input rows staged for a tile of 64 output pixels (at most)
  int vpitch;            // halo kernel: > 0, lanes take consecutive cells of output rows this wide
  // convolution epilogue (null / 0: none): bias per output channel, then the
  // activation (1: ReLU), then the residual at the output's own position
  const float *bias, *res;
  int act;
};

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1.
// Every lambda of the kernels is forced inline: a lambda left as a call
// takes its captures by address, which puts the kernel's arguments in
// scratch memory and its buffer descriptors in vector registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// body(t, j) for t = first .. end - 1, j = std::integral_constant of
// (t - first) % U: a loop over whole groups of U with no branch inside its
// body, then the last partial group, guarded.  A ring of loads whose slot
// is (t - first) % U keeps its depth this way: with a guarded body inside
// the loop, the compiler's count of the loads in flight at each join is the
// smallest over its paths, and it waits for every load there.
template <int U, class F>
__device__ __forceinline__ void ring_loop(int first, int end, F &&body) {
  int t0 = first;
  for (; t0 + U <= end; t0 += U)
    static_for<U>([&](auto j) __attribute__((always_inline)) { body(t0 + decltype(j)::value, j); });
  static_for<U>([&](auto j) __attribute__((always_inline)) {
    if (t0 + decltype(j)::value < end) body(t0 + decltype(j)::value, j);
  });
}

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

// The sign mask of a staged tap: 0x80000000 for a tap at or beyond k (its
// padding +0 becomes -0 by an OR), 0 for a real tap.
__device__ __forceinline__ uint32_t pad_sign(bool past) { return past ? 0x80000000u : 0u; }
__device__ __forceinline__ float or_sign(float v, uint32_t sign) {
  return __uint_as_float(__float_as_uint(v) | sign);
}

// The value stored for output channel ch at dst: the finished sum, then the
// convolution epilogue of "Convolution (fast mode)", sections "Tiles and
// chunks" (bias, then activation) and "Single-column products" (bias,
// activation and residual) -- each a separately rounded operation after the
// whole sum, so the sum's bits are those of the plain convolution -- then a
// NaN made canonical.  ReLU keeps a NaN and turns every other value not
// above zero into +0.  The channel is a 32-bit index: computed in 64 bits
// (group * M + row) it made the compiler treat the tile bases of the staging
// loads as divergent, and the main loop read its operands through waterfall
// loops.
// EPI false: the plain store (kernels compiled both ways keep their store
// loops free of the epilogue's tests).
template <bool EPI = true>
__device__ __forceinline__ float finish(const Problem &p, float acc, int ch, const float *dst) {
  if constexpr (!EPI) return canonical(acc);
  float v = acc;
  if (p.bias != nullptr) v = v + p.bias[ch];
  if (p.act == 1) v = v > 0.0f ? v : (v != v ? v : 0.0f);
  if (p.res != nullptr) v = v + p.res[dst - p.C];
  return canonical(v);
}

// The epilogue on preloaded operands: b = bias[ch], r = the residual at the
// output's position, both read before any of the block's stores (a load
// after a store to a possibly equal address would wait for each in turn).
__device__ __forceinline__ float finish_with(const Problem &p, float acc, float b, float r) {
  float v = acc;
  if (p.bias != nullptr) v = v + b;
  if (p.act == 1) v = v > 0.0f ? v : (v != v ? v : 0.0f);
  if (p.res != nullptr) v = v + r;
  return canonical(v);
}
__device__ __forceinline__ float epi_bias(const Problem &p, bool ok, int ch) {
  return p.bias != nullptr && ok ? p.bias[ch] : 0.0f;
}
__device__ __forceinline__ float epi_res(const Problem &p, bool ok, const float *dst) {
  return p.res != nullptr && ok ? p.res[dst - p.C] : 0.0f;
}

// ---------------------------------------------------------------------------
// Loads.  Every staged operand is read with raw buffer loads: a 32-bit byte
// offset from a base held in scalar registers.  A load whose element lies
// outside the problem uses the offset kOutside, beyond the buffer's range,
// and the hardware returns +0 for it; no select after the load, and no
// branch around it, so every chunk issues the same loads and the waits for
// them can be counted exactly D-1 chunks later.
// ---------------------------------------------------------------------------
// kOutside + 16 must not wrap around 2^32, or a 16-byte load would pass the
// range check.
constexpr uint32_t kRange = 0xFFFFFF00u;    // range of a staging buffer, in bytes
constexpr uint32_t kOutside = kRange;       // an offset at or past the range: the load returns +0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
// The whole vector is reinterpreted before its elements are taken: taking
// them one by one from the integer vector made this compiler shrink the load
// to a single dword.
__device__ __forceinline__ void load3(__amdgpu_buffer_rsrc_t rs, uint32_t off, float *r) {
  typedef float f32x3 __attribute__((ext_vector_type(3)));
  const f32x3 v = __builtin_bit_cast(f32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0));
  r[0] = v.x;
  r[1] = v.y;
  r[2] = v.z;
}

__device__ __forceinline__ void load4(__amdgpu_buffer_rsrc_t rs, uint32_t off, float *r) {
  const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  r[0] = v.x;
  r[1] = v.y;
  r[2] = v.z;
  r[3] = v.w;
}

// ---------------------------------------------------------------------------
// A staging: rows of A (k contiguous), BM rows x BK taps per chunk, into a
// k-major LDS tile As[kk*LDA + row].  VEC: 16-byte loads of 4 taps (A
// 16-byte aligned, lda, the group stride and K multiples of 4, so a load is
// wholly inside or wholly outside the problem).
// ---------------------------------------------------------------------------
// OPB: the same staging for a B operand given as its transpose (N x K
// row-major, k contiguous like A's rows): BM columns of B per chunk, stored
// k-major as Bs[kk*LDB + col].
template <int BM, int BK, int NT, bool VEC, bool OPB = false>
struct AStage {
  static constexpr int KV = VEC ? 4 : 1;      // taps per load
  static constexpr int LPR = BK / KV;         // loads per row and chunk
  static constexpr int RSTEP = NT / LPR;      // rows between a thread's loads
  static constexpr int NQ = BM / RSTEP;       // loads per thread and chunk
  static constexpr int kRegs = NQ * KV;
  static_assert(NT % LPR == 0 && BM % RSTEP == 0 && NQ >= 1, "A staging shape");

  const float *blk;     // A_g row m0, tap 0
  uint32_t voff[NQ];    // byte offset of (row r0 + q*RSTEP, tap kc) from blk; kOutside past M
  int kc, r0;

  __device__ void init(const Problem &p, int g, int m0, int tid) {
    kc = (tid % LPR) * KV;
    r0 = tid / LPR;
    const int64_t ld = OPB ? p.ldb : p.lda;
    const int lim = OPB ? p.N : p.M;
    blk = OPB ? p.B + (int64_t)m0 * ld : p.A + g * p.a_gstride + (int64_t)m0 * ld;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      voff[q] = m0 + r0 + q * RSTEP < lim ? (uint32_t)(4 * ((r0 + q * RSTEP) * ld + kc))
                                          : kOutside;
  }
  __device__ void load(const Problem &p, int k0, float (&r)[kRegs]) const {
    const __amdgpu_buffer_rsrc_t rs = buffer_at(blk + k0, kRange);
    const bool kin = k0 + kc < p.K;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t o = kin ? voff[q] : kOutside;
      if (VEC)
        load4(rs, o, &r[q * 4]);
      else
        r[q] = load1(rs, o);
    }
  }
  template <int LDA>
  __device__ void store(float *lds, const float (&r)[kRegs]) const {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < KV; ++e) lds[(kc + e) * LDA + r0 + q * RSTEP] = r[q * KV + e];
  }
  // The same for the chunk starting at tap k0, this thread's taps at or
  // beyond K stored as -0 (pad_sign; VEC: K is a multiple of 4, so a load is
  // wholly inside or wholly past K).
  template <int LDA>
  __device__ void store_signed(float *lds, const float (&r)[kRegs], int k0, int K) const {
    const uint32_t sg = pad_sign(k0 + kc >= K);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int e = 0; e < KV; ++e)
        lds[(kc + e) * LDA + r0 + q * RSTEP] = or_sign(r[q * KV + e], sg);
  }
};

// ---------------------------------------------------------------------------
// B staging: BK taps x BN columns per chunk into Bs[kk*BN + col].
//  * matrix, VEC: 16-byte loads of 4 columns (B 16-byte aligned, ldb and N
//    multiples of 4);
//  * matrix scalar, planes, gather: thread -> one column and TPG consecutive
//    taps.  The gather decodes its first tap (c, ky, kx) once per chunk with
//    wave-uniform (scalar) arithmetic and steps the following taps
//    incrementally; a tap outside the input plane reads +0.
// ---------------------------------------------------------------------------
template <int BN, int BK, int NT, int KIND, bool VEC>
struct BStage {
  static constexpr bool V = VEC && KIND == kBMatrix;
  static constexpr int C4 = BN / 4;                       // float4 per k-row
  static constexpr int VRSTEP = V ? NT / C4 : 1;          // k-rows between a thread's loads
  static constexpr int VNQ = V ? BK / VRSTEP : 1;
  static constexpr int TPG = BK * BN / NT;                // scalar: taps per thread
  static constexpr int NV = V ? VNQ : (KIND == kBMatrix ? TPG : 1);
  static constexpr int kRegs = V ? VNQ * 4 : TPG;
  static_assert(V ? (NT % C4 == 0 && BK % VRSTEP == 0) : (NT % BN == 0 && TPG >= 1),
                "B staging shape");

  int col, t0;        // column in the tile; first tap (scalar) or k-row (vector) of this thread
  bool col_ok;
  const float *base;  // matrix: B + n0; conv: x + g*x_grp
  uint32_t voff[NV];  // matrix: byte offsets of this thread's elements of a chunk; kOutside past N
  int e0;             // conv: element offset of this column's (image, window origin) in base
  int iy0, ix0;       // gather: window origin of this column's output pixel

  __device__ void init(const Problem &p, int g, int n0, int tid) {
    if (V) {
      col = 4 * (tid % C4);
      t0 = tid / C4;
      col_ok = n0 + col < p.N;
      base = p.B + n0;
#pragma unroll
      for (int q = 0; q < VNQ; ++q)
        voff[q] = col_ok ? (uint32_t)(4 * ((t0 + q * VRSTEP) * p.ldb + col)) : kOutside;
      return;
    }
    col = tid % BN;
    t0 = __builtin_amdgcn_readfirstlane((tid / BN) * TPG);  // wave-uniform (BN >= 64)
    const int j = n0 + col;
    col_ok = j < p.N;
    if (KIND == kBMatrix) {
      base = p.B + n0;
#pragma unroll
      for (int q = 0; q < TPG; ++q)
        voff[q] = col_ok ? (uint32_t)(4 * ((t0 + q) * p.ldb + col)) : kOutside;
      return;
    }
    const int jj = col_ok ? j : 0;
    const int img = jj / p.OHW;
    const int pix = jj - img * p.OHW;
    base = p.B + g * p.x_grp;
    if (KIND == kBPlanes) {
      e0 = (int)(img * p.x_img) + pix;
    } else {
      const int oy = pix / p.OW;
      const int ox = pix - oy * p.OW;
      iy0 = oy * p.sH - p.pT;
      ix0 = ox * p.sW - p.pL;
      e0 = (int)(img * p.x_img) + iy0 * p.W + ix0;
    }
  }

  __device__ void load(const Problem &p, int k0, float (&r)[kRegs]) const {
    if (V) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(base + (int64_t)k0 * p.ldb, kRange);
#pragma unroll
      for (int q = 0; q < VNQ; ++q)
        load4(rs, k0 + t0 + q * VRSTEP < p.K ? voff[q] : kOutside, &r[q * 4]);
      return;
    }
    const int t = k0 + t0;  // first tap of this thread (wave-uniform)
    if (KIND == kBMatrix) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(base + (int64_t)k0 * p.ldb, kRange);
#pragma unroll
      for (int q = 0; q < TPG; ++q) r[q] = load1(rs, t + q < p.K ? voff[q] : kOutside);
      return;
    }
    const __amdgpu_buffer_rsrc_t rs = buffer_at(base, kRange);
    if (KIND == kBPlanes) {
#pragma unroll
      for (int q = 0; q < TPG; ++q) {
        const bool ok = col_ok && t + q < p.K;  // plane t+q of the group
        r[q] = load1(rs, ok ? (uint32_t)(4 * (e0 + (t + q) * p.HW)) : kOutside);
      }
      return;
    }
    // gather: tap t -> (c, ky, kx) once, then step through the following taps
    int c = t / p.KHW;
    const int rr = t - c * p.KHW;
    int ky = rr / p.KW;
    int kx = rr - ky * p.KW;
#pragma unroll
    for (int q = 0; q < TPG; ++q) {
      const int dy = ky * p.dH, dx = kx * p.dW;
      const bool ok = col_ok && t + q < p.K && (unsigned)(iy0 + dy) < (unsigned)p.H &&
                      (unsigned)(ix0 + dx) < (unsigned)p.W;  // outside the plane: padding, +0
      r[q] = load1(rs, ok ? (uint32_t)(4 * (e0 + c * p.HW + dy * p.W + dx)) : kOutside);
      if (++kx == p.KW) {
        kx = 0;
        if (++ky == p.KH) {
          ky = 0;
          ++c;
        }
      }
    }
  }

  __device__ void store(float *lds, const float (&r)[kRegs]) const {
    if (V) {
#pragma unroll
      for (int q = 0; q < VNQ; ++q)
        *reinterpret_cast<float4 *>(&lds[(t0 + q * VRSTEP) * BN + col]) =
            make_float4(r[q * 4 + 0], r[q * 4 + 1], r[q * 4 + 2], r[q * 4 + 3]);
      return;
    }
#pragma unroll
    for (int q = 0; q < TPG; ++q) lds[(t0 + q) * BN + col] = r[q];
  }
  // The same for the chunk starting at tap k0, taps at or beyond K stored as
  // -0 (pad_sign).
  __device__ void store_signed(float *lds, const float (&r)[kRegs], int k0, int K) const {
    if (V) {
#pragma unroll
      for (int q = 0; q < VNQ; ++q) {
        const uint32_t sg = pad_sign(k0 + t0 + q * VRSTEP >= K);
        *reinterpret_cast<float4 *>(&lds[(t0 + q * VRSTEP) * BN + col]) =
            make_float4(or_sign(r[q * 4 + 0], sg), or_sign(r[q * 4 + 1], sg),
                        or_sign(r[q * 4 + 2], sg), or_sign(r[q * 4 + 3], sg));
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < TPG; ++q) lds[(t0 + q) * BN + col] = or_sign(r[q], pad_sign(k0 + t0 + q >= K));
  }
};

// Pointer to output (row, col) of group g.
template <int KIND>
__device__ inline float *out_ptr(const Problem &p, int g, int row, int col) {
  if (KIND == kBMatrix || KIND == kBMatrixT) return p.C + (int64_t)row * p.ldc + col;
  const int img = col / p.OHW;
  const int pix = col - img * p.OHW;
  return p.C + img * p.y_img + g * p.y_grp + (int64_t)row * p.OHW + pix;
}

// ---------------------------------------------------------------------------
// The staging pipeline.  Chunk c's loads go to register slot c % D, D-1
// chunks ahead of its use; at its turn the slot is written to LDS buffer
// c % 2 (store(slot, buffer, c)), one barrier, then the chunk's products.
// One barrier per chunk is
// enough with two LDS buffers: a wave writing buffer c % 2 has passed the
// barrier of chunk c-1, so every wave has finished reading chunk c-2 there.
// The main loop runs whole groups of D chunks and issues every load
// unconditionally (past the last chunk it reloads the last one), so each
// wait is for loads issued D-1 chunks earlier; the remaining chunks are
// consumed without further loads.
// ---------------------------------------------------------------------------
template <int D, class Load, class Store, class Compute>
__device__ __forceinline__ void run_pipeline(int nchunks, Load &&load, Store &&store,
                                             Compute &&compute) {
  static_assert(D >= 2 && D % 2 == 0, "pipeline depth");
  if (nchunks <= 0) return;
  const int last = nchunks - 1;
  static_for<D - 1>([&](auto j) __attribute__((always_inline)) { load(min((int)decltype(j)::value, last), j); });
  const int full = nchunks - nchunks % D;
  for (int c0 = 0; c0 < full; c0 += D) {
    static_for<D>([&](auto j) __attribute__((always_inline)) {
      constexpr int J = decltype(j)::value;
      load(min(c0 + J + D - 1, last), std::integral_constant<int, (J + D - 1) % D>{});
      store(j, std::integral_constant<int, J % 2>{}, c0 + J);
      __syncthreads();
      compute(c0 + J, std::integral_constant<int, J % 2>{}, j);
    });
  }
  static_for<D - 1>([&](auto j) __attribute__((always_inline)) {
    constexpr int J = decltype(j)::value;
    if (full + J < nchunks) {
      store(j, std::integral_constant<int, J % 2>{}, full + J);
      __syncthreads();
      compute(full + J, std::integral_constant<int, J % 2>{}, j);
    }
  });
}

// ---------------------------------------------------------------------------
// Matrix-core kernel.  4 or 8 waves arranged WM x WN; a wave owns a
// (TM*32) x (TN*64) sub-tile as TM x TN blocks of 32 x 64 outputs, each block
// one 32x32x1 MFMA pair-of-blocks: lanes 0-31 and 32-63 both carry the 32 A
// rows, lanes 0-31 carry B columns 0-31 and lanes 32-63 columns 32-63.
// ---------------------------------------------------------------------------
// One k step of an MF x 64 block: D = a (x) b + c, one fused multiply-add
// per element (32x32x1 two-block or 16x16x1 four-block fp32 MFMA).
template <int MF>
__device__ __forceinline__ std::conditional_t<MF == 32, f32x32, f32x16> mfma1(
    float a, float b, std::conditional_t<MF == 32, f32x32, f32x16> c) {
  if constexpr (MF == 32)
    return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, c, 0, 0, 0);
}

template <int MODE, int BM, int BN, int WM, int WN, int KIND, bool AVEC, bool BVEC, int D,
          int MF = 32>
__global__ void __launch_bounds__(64 * WM * WN) mfma_kernel(Problem p) {
  constexpr int NT = 64 * WM * WN, BK = 16;
  constexpr int TM = BM / WM / MF, TN = BN / WN / 64;
  static_assert((WM * WN == 4 || WM * WN == 8) && TM >= 1 && TN >= 1, "tile shape");
  // MF = 16: blocks of 16 x 64 outputs, one v_mfma_f32_16x16x1_4b_f32 per k
  // (its four 16x16 blocks share the 16 A rows)
  static_assert(MF == 32 || MF == 16, "block rows");
  using acc_t = std::conditional_t<MF == 32, f32x32, f32x16>;
  constexpr int LDA = BM + 1;  // k-major A tile, padded against bank conflicts of the transposing store
  // a transposed B (N x K) is staged like A, its k-major tile padded by 4
  constexpr bool BT = KIND == kBMatrixT;
  constexpr int LDB = BT ? BN + 4 : BN;
  __shared__ __align__(16) float As[2][BK * LDA];
  __shared__ __align__(16) float Bs[2][BK * LDB];
  // 16-byte loads only where every thread has at least one of them
  using AS = AStage<BM, BK, NT, AVEC && (BM * BK / 4 >= NT)>;
  using BS = std::conditional_t<BT, AStage<BN, BK, NT, BVEC && (BN * BK / 4 >= NT), true>,
                                BStage<BN, BK, NT, BT ? kBMatrix : KIND, BVEC && (BN * BK / 4 >= NT)>>;

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  AS as;
  BS bs;
  as.init(p, tc.g, m0, tid);
  bs.init(p, tc.g, n0, tid);
  float ra[D][AS::kRegs];
  float rb[D][BS::kRegs];

  acc_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
  // Exact mode, matrix B and input planes: the rounded products of the last
  // two k steps (k % 2), a step's products added while the next step's are
  // made.  Exact mode with gathered B: the last product made, added one
  // MFMA later (two steps of products beside the gather's registers do not
  // fit two waves per SIMD).
  constexpr bool kPend = MODE == kExact && KIND == kBGather;
  constexpr int NPB = MODE == kExact && !kPend ? 2 : 1;
  acc_t prod[NPB][TM][TN];
#pragma unroll
  for (int u = 0; u < NPB; ++u)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) prod[u][i][j] = acc_t{};
  acc_t pend = acc_t{};

  const int a_off = wm * TM * MF + (lane & (MF - 1));
  const int b_off = wn * TN * 64 + lane;

  run_pipeline<D>(
      (p.K + BK - 1) / BK,
      [&](int c, auto slot) __attribute__((always_inline)) {
        as.load(p, c * BK, ra[decltype(slot)::value]);
        bs.load(p, c * BK, rb[decltype(slot)::value]);
      },
      [&](auto slot, auto buf, int c) __attribute__((always_inline)) {
        // fast mode: the A tile's taps past K are -0 (B's are +0).  Only the
        // chunk that runs past K has such taps: a uniform test skips the sign
        // fix elsewhere, except where a wave holds 2 x 2 blocks (the 128 x 256
        // and 256 x 256 tiles), whose branch-free form measured faster
        // (4096^3 on 256 x 256: 0.986 ms against 0.999 with the test;
        // 2048 x 11008 x 4096 on 128 x 256: 1.54 against 1.99 ms), while the
        // test made the 64 x 128 tile's 512 x 11008 x 4096 launch 416 -> 408 us
        constexpr bool kSignTest = TM * TN < 4;
        if (MODE == kFast && (!kSignTest || (c + 1) * BK > p.K))
          as.template store_signed<LDA>(As[decltype(buf)::value], ra[decltype(slot)::value], c * BK,
                                        p.K);
        else
          as.template store<LDA>(As[decltype(buf)::value], ra[decltype(slot)::value]);
        if constexpr (BT)
          bs.template store<LDB>(Bs[decltype(buf)::value], rb[decltype(slot)::value]);
        else
          bs.store(Bs[decltype(buf)::value], rb[decltype(slot)::value]);
      },
      [&](int, auto buf, auto) __attribute__((always_inline)) {
        const float *al = As[decltype(buf)::value];
        const float *bl = Bs[decltype(buf)::value];
        if constexpr (kPend) {
          // a rolled k loop, so only one k's products are live at a time
#pragma unroll 2
          for (int kk = 0; kk < BK; ++kk) {
            float a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = al[kk * LDA + a_off + i * MF];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[j] = bl[kk * LDB + b_off + j * 64];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j) {
                const acc_t pr = mfma1<MF>(a[i], b[j], acc_t{});
                const int s = i * TN + j;  // the product before this one: block s - 1
                const int pi = s == 0 ? TM - 1 : (s - 1) / TN;
                const int pj = s == 0 ? TN - 1 : (s - 1) % TN;
                acc[pi][pj] += pend;  // the first pend is +0: acc stays +0
                pend = pr;
              }
          }
          return;
        } else if constexpr (MODE == kExact) {
          // Exact: per k the MFMAs form this k's rounded products (C = +0)
          // in one product buffer while the VALU adds the previous k's
          // products, from the other buffer, into the accumulators: the
          // matrix pipe and the VALU work at the same time.  The add of a
          // product waits a whole k step, past the MFMA's latency.  (The
          // first adds take the zero-initialised buffer: acc stays +0.)
          // Operands are read RA k steps ahead (ring of RA + 1), so a
          // step's LDS reads have a whole step of adds to return.
          constexpr int RA = 2;
          float a[RA + 1][TM], b[RA + 1][TN];
          static_for<RA>([&](auto rq) __attribute__((always_inline)) {
            constexpr int R0 = decltype(rq)::value;
#pragma unroll
            for (int i = 0; i < TM; ++i) a[R0][i] = al[R0 * LDA + a_off + i * MF];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[R0][j] = bl[R0 * LDB + b_off + j * 64];
          });
          auto step = [&](auto uq, auto kq) __attribute__((always_inline)) {
            constexpr int U = decltype(uq)::value, KK = decltype(kq)::value;
            constexpr int S = KK % (RA + 1), SN = (KK + RA) % (RA + 1);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                prod[U][i][j] = mfma1<MF>(a[S][i], b[S][j], acc_t{});
            if constexpr (KK + RA < BK) {
#pragma unroll
              for (int i = 0; i < TM; ++i) a[SN][i] = al[(KK + RA) * LDA + a_off + i * MF];
#pragma unroll
              for (int j = 0; j < TN; ++j) b[SN][j] = bl[(KK + RA) * LDB + b_off + j * 64];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j) acc[i][j] += prod[U ^ 1][i][j];
            __builtin_amdgcn_sched_barrier(0);
          };
          static_for<BK>([&](auto kq) __attribute__((always_inline)) {
            constexpr int KK = decltype(kq)::value;
            step(std::integral_constant<int, KK & 1>{}, kq);
          });
          return;
        }
        float a[2][TM], b[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[0][i] = al[a_off + i * MF];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[0][j] = bl[b_off + j * 64];
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
          const int u = kk & 1;
          if (kk + 1 < BK) {  // operands of the next k, read while this k's MFMAs run
#pragma unroll
            for (int i = 0; i < TM; ++i) a[u ^ 1][i] = al[(kk + 1) * LDA + a_off + i * MF];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[u ^ 1][j] = bl[(kk + 1) * LDB + b_off + j * 64];
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = mfma1<MF>(a[u][i], b[u][j], acc[i][j]);
        }
      });
  if constexpr (kPend) {
    acc[TM - 1][TN - 1] += pend;
  } else if constexpr (MODE == kExact) {
    // the products of the last k (BK is even: they sit in buffer 1)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += prod[NPB - 1][i][j];
  }

  // The stores, with the convolution epilogue or without it: one uniform test
  // picks the loop, so a plain product's stores carry no per-output tests
  // (those slowed the store-bound 1x1 convolutions by up to 20 %).
  auto store_all = [&](auto epi) __attribute__((always_inline)) {
    constexpr bool E = decltype(epi)::value;
    if constexpr (MF == 16) {
      // Epilogue of the 16 x 64 blocks: register r of lane l holds row
      // 4*(l/16) + r%4 and column 16*(r/4) + l%16 (measured on gfx950).
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
        {
          float pb[16], pr[16];
          if constexpr (E) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int col = n0 + wn * TN * 64 + j * 64 + 16 * (r >> 2) + (lane & 15);
              const int row = m0 + wm * TM * 16 + i * 16 + 4 * (lane >> 4) + (r & 3);
              const bool ok = col < p.N && row < p.M;
              pb[r] = epi_bias(p, ok, tc.g * p.M + row);
              pr[r] = epi_res(p, ok, ok ? out_ptr<KIND>(p, tc.g, row, col) : p.C);
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int col = n0 + wn * TN * 64 + j * 64 + 16 * (r >> 2) + (lane & 15);
            const int row = m0 + wm * TM * 16 + i * 16 + 4 * (lane >> 4) + (r & 3);
            if (col < p.N && row < p.M) {
              float *d = out_ptr<KIND>(p, tc.g, row, col);
              if constexpr (E)
                *d = finish_with(p, acc[i][j][r], pb[r], pr[r]);
              else
                *d = finish<false>(p, acc[i][j][r], 0, d);
            }
          }
        }
      return;
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
          const int64_t rstride = KIND == kBMatrix || KIND == kBMatrixT ? p.ldc : (int64_t)p.OHW;
          float pb[16], pr[16];
          if constexpr (E) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = m0 + wm * TM * 32 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
              pb[r] = epi_bias(p, row < p.M, tc.g * p.M + row);
              pr[r] = epi_res(p, row < p.M, base + (row < p.M ? row : 0) * rstride);
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * TM * 32 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
            if (row < p.M) {
              if constexpr (E)
                base[row * rstride] = finish_with(p, acc[i][j][h * 16 + r], pb[r], pr[r]);
              else
                base[row * rstride] = finish<false>(p, acc[i][j][h * 16 + r], 0, base);
            }
          }
        }
  };
  if (p.bias == nullptr && p.res == nullptr && p.act == 0)
    store_all(std::false_type{});
  else
    store_all(std::true_type{});
}

// ---------------------------------------------------------------------------
// VALU kernel: 64 x 64 tile, 256 threads in a 16 x 16 grid, each thread a
// 4 x 4 micro-tile (rows ty*4.., columns tx*4..).  Per term: v_fma_f32 in fast
// mode, v_mul_f32 then v_add_f32 in exact mode.
// ---------------------------------------------------------------------------
template <int MODE, int KIND>
__global__ void __launch_bounds__(256) valu_kernel(Problem p) {
  constexpr int NT = 256, BK = 16, BM = 64, BN = 64, D = 2;
  constexpr int LDA = BM + 4;
  __shared__ __align__(16) float As[2][BK * LDA];
  constexpr bool BT = KIND == kBMatrixT;  // a transposed B is staged like A
  constexpr int LDB = BT ? BN + 4 : BN;
  __shared__ __align__(16) float Bs[2][BK * LDB];
  using AS = AStage<BM, BK, NT, false>;
  using BS = std::conditional_t<BT, AStage<BN, BK, NT, false, true>,
                                BStage<BN, BK, NT, BT ? kBMatrix : KIND, false>>;

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  AS as;
  BS bs;
  as.init(p, tc.g, m0, tid);
  bs.init(p, tc.g, n0, tid);
  float ra[D][AS::kRegs];
  float rb[D][BS::kRegs];

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  run_pipeline<D>(
      (p.K + BK - 1) / BK,
      [&](int c, auto slot) __attribute__((always_inline)) {
        as.load(p, c * BK, ra[decltype(slot)::value]);
        bs.load(p, c * BK, rb[decltype(slot)::value]);
      },
      [&](auto slot, auto buf, int c) __attribute__((always_inline)) {
        // fast mode: the A tile's taps past K are -0 (B's are +0); only the
        // chunk that runs past K has such taps (a uniform test)
        if (MODE == kFast && (c + 1) * BK > p.K)
          as.template store_signed<LDA>(As[decltype(buf)::value], ra[decltype(slot)::value], c * BK,
                                        p.K);
        else
          as.template store<LDA>(As[decltype(buf)::value], ra[decltype(slot)::value]);
        if constexpr (BT)
          bs.template store<LDB>(Bs[decltype(buf)::value], rb[decltype(slot)::value]);
        else
          bs.store(Bs[decltype(buf)::value], rb[decltype(slot)::value]);
      },
      [&](int, auto buf, auto) __attribute__((always_inline)) {
        const float *al = As[decltype(buf)::value];
        const float *bl = Bs[decltype(buf)::value];
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
          const float4 a4 = *reinterpret_cast<const float4 *>(&al[kk * LDA + ty * 4]);
          const float4 b4 = *reinterpret_cast<const float4 *>(&bl[kk * LDB + tx * 4]);
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
      });
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + tx * 4 + j;
    if (col >= p.N) continue;
    float *base = out_ptr<KIND>(p, tc.g, 0, col);
    const int64_t rstride = KIND == kBMatrix || KIND == kBMatrixT ? p.ldc : (int64_t)p.OHW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      if (row < p.M) base[row * rstride] = finish(p, acc[i][j], tc.g * p.M + row, base + row * rstride);
    }
  }
}

// One term for every lane, with the weight taken from lane U of the lane's
// row of 16 (DPP row_newbcast on the first source operand), in one VOP2
// instruction: fast mode v_fmac_f32 (acc += w*b, one rounding); exact mode
// v_mul_f32 (the rounded product), then a separately rounded add.  The
// weight register is written only by memory loads, never by a VALU
// instruction, so the DPP read has no VALU-write hazard to wait out.
template <int MODE, int U>
__device__ __forceinline__ float step_bcast(float acc, float w, float b) {
  if (MODE == kFast) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "+v"(acc)
        : "v"(w), "v"(b), "n"(U));
    return acc;
  } else {
    float prod;
    asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
        : "=v"(prod)
        : "v"(w), "v"(b), "n"(U));
    return acc + prod;
  }
}

// ---------------------------------------------------------------------------
// Lane kernel, for shapes with few outputs and long k (the deep layers of a
// convolution network at batch 1, short matrix products): a 32x32x1 MFMA
// takes 64 cycles per dependent k step, a VALU fused multiply-add about 5.
// Lane l of a wave owns output column n0 + l for the wave's R output rows.
// The B value of a k step comes from the LDS tile all W waves of the block
// share; the weight of a step is the same for every lane: a register holds
// 16 taps of a row (lane l: tap l % 16, the same in each row of 16 lanes)
// and a DPP row broadcast hands tap kk to all lanes.  Weights and B tiles
// are loaded D-1 chunks ahead.
// ---------------------------------------------------------------------------
// (Matrix operands with one or two rows per wave: at least 6 waves per SIMD.
// Left free, the compiler gave the exact two-row form 106 registers and 4
// waves where 70 registers suffice; the ragged exact product ran 8 % slower.)
template <int MODE, int KIND, int R, int W, int D>
__global__ void __launch_bounds__(64 * W)
    __attribute__((amdgpu_waves_per_eu(KIND == kBMatrix && R <= 2 ? 6 : 1))) lane_kernel(Problem p) {
  constexpr int NT = 64 * W, BK = 32, BN = 64, WR = BK / 16;
  __shared__ __align__(16) float Bs[2][BK * BN];
  using BS = BStage<BN, BK, NT, KIND, false>;

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = tc.tn * BN;
  const int row0 = tc.tm * (R * W) + wave * R;

  BS bs;
  bs.init(p, tc.g, n0, tid);
  float rb[D][BS::kRegs];
  float wv[D][R][WR];

  // Weight row per output row (a row beyond M reads row M-1, never stored).
  const float *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.M - 1);
    wrow[r] = p.A + tc.g * p.a_gstride + (int64_t)row * p.lda;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  run_pipeline<D>(
      (p.K + BK - 1) / BK,
      [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        const int k0 = c * BK;
        bs.load(p, k0, rb[S]);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int h = 0; h < WR; ++h) {
            const int t = 16 * h + (lane & 15);
            wv[S][r][h] = load1(buffer_at(wrow[r] + k0, kRange),
                                k0 + t < p.K ? (uint32_t)(4 * t) : kOutside);
          }
      },
      [&](auto slot, auto buf, int c) __attribute__((always_inline)) {
        // fast mode: B's taps past K are -0 (the weight registers hold +0
        // there: they are read through DPP and never written by the VALU);
        // only the chunk that runs past K has such taps (a uniform test)
        if (MODE == kFast && (c + 1) * BK > p.K)
          bs.store_signed(Bs[decltype(buf)::value], rb[decltype(slot)::value], c * BK, p.K);
        else
          bs.store(Bs[decltype(buf)::value], rb[decltype(slot)::value]);
      },
      [&](int, auto buf, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        const float *bl = Bs[decltype(buf)::value];
        // the chunk's B values first, all issued before the chains (the
        // scheduling barrier keeps the compiler from sinking each read to
        // just before its use, where its latency would stall the chain)
        float bv[BK];
        static_for<BK>([&](auto kk) __attribute__((always_inline)) {
          constexpr int KK = decltype(kk)::value;
          bv[KK] = bl[KK * BN + lane];
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<BK>([&](auto kk) __attribute__((always_inline)) {
          constexpr int KK = decltype(kk)::value;
#pragma unroll
          for (int r = 0; r < R; ++r)
            acc[r] = step_bcast<MODE, KK % 16>(acc[r], wv[S][r][KK / 16], bv[KK]);
        });
      });
  const int col = n0 + lane;
  if (col < p.N) {
    float *base = out_ptr<KIND>(p, tc.g, 0, col);
    const int64_t rstride = KIND == kBMatrix ? p.ldc : (int64_t)p.OHW;
    // one uniform test picks the store loop with or without the epilogue;
    // with it, the rows' biases and residuals are loaded before the stores
    auto store_all = [&](auto epi) __attribute__((always_inline)) {
      constexpr bool E = decltype(epi)::value;
      float pb[R], pr[R];
      if constexpr (E) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool ok = row0 + r < p.M;
          pb[r] = epi_bias(p, ok, tc.g * p.M + row0 + r);
          pr[r] = epi_res(p, ok, base + (ok ? row0 + r : 0) * rstride);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (row0 + r < p.M) {
          if constexpr (E)
            base[(row0 + r) * rstride] = finish_with(p, acc[r], pb[r], pr[r]);
          else
            base[(row0 + r) * rstride] = finish<false>(p, acc[r], 0, base);
        }
    };
    if (p.bias == nullptr && p.res == nullptr && p.act == 0)
      store_all(std::false_type{});
    else
      store_all(std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// Lane kernel for a KH x KW convolution known at compile time.  The columns
// of a block are 64 output pixels of one image.  A k-chunk is CC whole input
// channels (CC*KH*KW taps; every wave stages CPW channels).  Each lane keeps,
// for every kernel position (ky, kx), the byte offset of its input pixel in
// a plane, or an offset beyond the plane when the tap falls in the padding;
// a tap's load then needs no arithmetic at all: a buffer load of the
// channel's plane at that offset, which reads +0 outside the plane.  The
// padding zeros are produced during the gather and never stored in memory.
// ---------------------------------------------------------------------------
template <int MODE, int KH, int KW, int R, int W, int D>
__global__ void __launch_bounds__(64 * W) lane_conv_kernel(Problem p) {
  constexpr int KHW = KH * KW;
  constexpr int CPW = KHW >= 32 ? 1 : (32 / KHW + W - 1) / W;  // channels per wave and chunk
  constexpr int CC = W * CPW;                                  // channels per chunk
  constexpr int BK = CC * KHW, BN = 64, WR = (BK + 15) / 16, PER = CPW * KHW;
  __shared__ __align__(16) float Bs[2][BK * BN];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tpi = (p.OHW + BN - 1) / BN;  // column tiles per image
  const int img = tc.tn / tpi;
  const int pix = (tc.tn - img * tpi) * BN + lane;
  const int row0 = tc.tm * (R * W) + wave * R;
  const int cin_g = p.K / KHW;

  // byte offsets of this lane's taps inside a plane
  uint32_t voff[KHW];
  {
    const bool valid = pix < p.OHW;
    const int oy = valid ? pix / p.OW : 0;
    const int ox = valid ? pix - oy * p.OW : 0;
    const int iy0 = oy * p.sH - p.pT, ix0 = ox * p.sW - p.pL;
#pragma unroll
    for (int ky = 0; ky < KH; ++ky)
#pragma unroll
      for (int kx = 0; kx < KW; ++kx) {
        const int iy = iy0 + ky * p.dH, ix = ix0 + kx * p.dW;
        const bool in = valid && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
        voff[ky * KW + kx] = in ? (uint32_t)(4 * (iy * p.W + ix)) : kOutside;
      }
  }
  const float *xg = p.B + img * p.x_img + tc.g * p.x_grp;  // channel 0 of (image, group)
  const int plane_bytes = 4 * p.HW;

  float rb[D][PER];
  float wv[D][R][WR];
  const float *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.M - 1);  // a row beyond M is computed, never stored
    wrow[r] = p.A + tc.g * p.a_gstride + (int64_t)row * p.lda;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  run_pipeline<D>(
      (cin_g + CC - 1) / CC,
      [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
          const int ch = c * CC + wave * CPW + cc;  // wave-uniform
          // a channel beyond K gets an empty range: its loads read +0
          const __amdgpu_buffer_rsrc_t rs = buffer_at(
              xg + (int64_t)min(ch, cin_g - 1) * p.HW, ch < cin_g ? (uint32_t)plane_bytes : 0u);
#pragma unroll
          for (int k = 0; k < KHW; ++k) rb[S][cc * KHW + k] = load1(rs, voff[k]);
        }
        const int k0 = c * BK;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int h = 0; h < WR; ++h) {
            const int t = 16 * h + (lane & 15);
            wv[S][r][h] = load1(buffer_at(wrow[r] + k0, kRange),
                                k0 + t < p.K ? (uint32_t)(4 * t) : kOutside);
          }
      },
      [&](auto slot, auto buf, int c) __attribute__((always_inline)) {
        float *bl = Bs[decltype(buf)::value];
        // fast mode: the taps of channels past the group's last are -0 (the
        // weights there are +0); only the chunk that runs past the group's
        // channels has such taps (a uniform test)
        if (MODE == kFast && (c + 1) * CC > cin_g) {
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc) {
            const uint32_t sg = pad_sign(c * CC + wave * CPW + cc >= cin_g);
#pragma unroll
            for (int k = 0; k < KHW; ++k)
              bl[(wave * PER + cc * KHW + k) * BN + lane] =
                  or_sign(rb[decltype(slot)::value][cc * KHW + k], sg);
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
            for (int k = 0; k < KHW; ++k)
              bl[(wave * PER + cc * KHW + k) * BN + lane] = rb[decltype(slot)::value][cc * KHW + k];
        }
      },
      [&](int, auto buf, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        const float *bl = Bs[decltype(buf)::value];
        // the chunk's B values first, all issued before the chains (the
        // scheduling barrier keeps the compiler from sinking each read to
        // just before its use, where its latency would stall the chain)
        float bv[BK];
        static_for<BK>([&](auto kk) __attribute__((always_inline)) {
          constexpr int KK = decltype(kk)::value;
          bv[KK] = bl[KK * BN + lane];
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<BK>([&](auto kk) __attribute__((always_inline)) {
          constexpr int KK = decltype(kk)::value;
#pragma unroll
          for (int r = 0; r < R; ++r)
            acc[r] = step_bcast<MODE, KK % 16>(acc[r], wv[S][r][KK / 16], bv[KK]);
        });
      });
  if (pix < p.OHW) {
    float *base = out_ptr<kBGather>(p, tc.g, 0, img * p.OHW + pix);
    // one uniform test picks the store loop with or without the epilogue
    auto store_all = [&](auto epi) __attribute__((always_inline)) {
      constexpr bool E = decltype(epi)::value;
      float pb[R], pr[R];
      if constexpr (E) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool ok = row0 + r < p.M;
          pb[r] = epi_bias(p, ok, tc.g * p.M + row0 + r);
          pr[r] = epi_res(p, ok, base + (int64_t)(ok ? row0 + r : 0) * p.OHW);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (row0 + r < p.M) {
          if constexpr (E)
            base[(int64_t)(row0 + r) * p.OHW] = finish_with(p, acc[r], pb[r], pr[r]);
          else
            base[(int64_t)(row0 + r) * p.OHW] = finish<false>(p, acc[r], 0, base);
        }
    };
    if (p.bias == nullptr && p.res == nullptr && p.act == 0)
      store_all(std::false_type{});
    else
      store_all(std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// Runs of 8 or 16 k steps of one or two rows in one asm block: the weight of
// step u comes from lane u of the lane's row of 16 (DPP row_newbcast).  A
// VALU write of a register read through DPP must be followed by two wait
// states before that read; the weight registers are normally written by
// loads, but the compiler may copy them (from AGPRs, say) on the VALU just
// before the block, so every block starts with s_nop 1.  Inside a block the
// DPP-read registers are never written.
//   fast : acc = fma(w[u], b[u], acc)                       (v_fmac_f32_dpp)
//   exact: p = round(w[u] * b[u]) (v_mul_f32_dpp); acc = round(acc + p); the
//          product of step u+1 is formed while the sum of step u is pending.
// ---------------------------------------------------------------------------
#define OG_DPP(u) " row_newbcast:" #u " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
// fast, one row: %0 acc, %1 weights, %2.. B values
#define OG_F1(u, b) "v_fmac_f32_dpp %0, %1, %" #b OG_DPP(u)
#define OG_FAST1_4 "s_nop 1\n" OG_F1(0, 2) OG_F1(1, 3) OG_F1(2, 4) OG_F1(3, 5)
#define OG_FAST1_8                                                                     \
  "s_nop 1\n" OG_F1(0, 2) OG_F1(1, 3) OG_F1(2, 4) OG_F1(3, 5) OG_F1(4, 6) OG_F1(5, 7) \
      OG_F1(6, 8) OG_F1(7, 9)
#define OG_FAST1_16                                                                   \
  OG_FAST1_8 OG_F1(8, 10) OG_F1(9, 11) OG_F1(10, 12) OG_F1(11, 13) OG_F1(12, 14) \
      OG_F1(13, 15) OG_F1(14, 16) OG_F1(15, 17)
// fast, two rows: %0 %1 acc, %2 %3 weights, %4.. B values
#define OG_F2(u, b) "v_fmac_f32_dpp %0, %2, %" #b OG_DPP(u) "v_fmac_f32_dpp %1, %3, %" #b OG_DPP(u)
#define OG_FAST2_4 "s_nop 1\n" OG_F2(0, 4) OG_F2(1, 5) OG_F2(2, 6) OG_F2(3, 7)
#define OG_FAST2_8                                                                      \
  "s_nop 1\n" OG_F2(0, 4) OG_F2(1, 5) OG_F2(2, 6) OG_F2(3, 7) OG_F2(4, 8) OG_F2(5, 9) \
      OG_F2(6, 10) OG_F2(7, 11)
#define OG_FAST2_16                                                                    \
  OG_FAST2_8 OG_F2(8, 12) OG_F2(9, 13) OG_F2(10, 14) OG_F2(11, 15) OG_F2(12, 16) \
      OG_F2(13, 17) OG_F2(14, 18) OG_F2(15, 19)
// exact, one row: %0 acc, %1 %2 products of even / odd steps, %3 weights,
// %4.. B values
#define OG_M1(t, u, b) "v_mul_f32_dpp %" #t ", %3, %" #b OG_DPP(u)
#define OG_A1(t) "v_add_f32 %0, %0, %" #t "\n"
#define OG_EXACT1_HEAD                                                                    \
  "s_nop 1\n" OG_M1(1, 0, 4) OG_M1(2, 1, 5) OG_A1(1) OG_M1(1, 2, 6) OG_A1(2) OG_M1(2, 3, 7) \
      OG_A1(1) OG_M1(1, 4, 8) OG_A1(2) OG_M1(2, 5, 9) OG_A1(1) OG_M1(1, 6, 10) OG_A1(2)     \
          OG_M1(2, 7, 11) OG_A1(1)
#define OG_EXACT1_8 OG_EXACT1_HEAD OG_A1(2)
#define OG_EXACT1_4 \
  "s_nop 1\n" OG_M1(1, 0, 4) OG_M1(2, 1, 5) OG_A1(1) OG_M1(1, 2, 6) OG_A1(2) OG_M1(2, 3, 7) OG_A1(1) OG_A1(2)
#define OG_EXACT1_16                                                                      \
  OG_EXACT1_HEAD OG_M1(1, 8, 12) OG_A1(2) OG_M1(2, 9, 13) OG_A1(1) OG_M1(1, 10, 14) OG_A1(2) \
      OG_M1(2, 11, 15) OG_A1(1) OG_M1(1, 12, 16) OG_A1(2) OG_M1(2, 13, 17) OG_A1(1)          \
          OG_M1(1, 14, 18) OG_A1(2) OG_M1(2, 15, 19) OG_A1(1) OG_A1(2)
// exact, two rows: %0 %1 acc, %2 %3 products of even steps, %4 %5 of odd
// steps, %6 %7 weights, %8.. B values
#define OG_M2(ta, tb, u, b) \
  "v_mul_f32_dpp %" #ta ", %6, %" #b OG_DPP(u) "v_mul_f32_dpp %" #tb ", %7, %" #b OG_DPP(u)
#define OG_A2(ta, tb) "v_add_f32 %0, %0, %" #ta "\n" "v_add_f32 %1, %1, %" #tb "\n"
#define OG_EXACT2_HEAD                                                                   \
  "s_nop 1\n" OG_M2(2, 3, 0, 8) OG_M2(4, 5, 1, 9) OG_A2(2, 3) OG_M2(2, 3, 2, 10)         \
      OG_A2(4, 5) OG_M2(4, 5, 3, 11) OG_A2(2, 3) OG_M2(2, 3, 4, 12) OG_A2(4, 5)          \
          OG_M2(4, 5, 5, 13) OG_A2(2, 3) OG_M2(2, 3, 6, 14) OG_A2(4, 5) OG_M2(4, 5, 7, 15) \
              OG_A2(2, 3)
#define OG_EXACT2_8 OG_EXACT2_HEAD OG_A2(4, 5)
#define OG_EXACT2_4                                                                          \
  "s_nop 1\n" OG_M2(2, 3, 0, 8) OG_M2(4, 5, 1, 9) OG_A2(2, 3) OG_M2(2, 3, 2, 10) OG_A2(4, 5) \
      OG_M2(4, 5, 3, 11) OG_A2(2, 3) OG_A2(4, 5)
#define OG_EXACT2_16                                                                     \
  OG_EXACT2_HEAD OG_M2(2, 3, 8, 16) OG_A2(4, 5) OG_M2(4, 5, 9, 17) OG_A2(2, 3)           \
      OG_M2(2, 3, 10, 18) OG_A2(4, 5) OG_M2(4, 5, 11, 19) OG_A2(2, 3) OG_M2(2, 3, 12, 20) \
          OG_A2(4, 5) OG_M2(4, 5, 13, 21) OG_A2(2, 3) OG_M2(2, 3, 14, 22) OG_A2(4, 5)     \
              OG_M2(4, 5, 15, 23) OG_A2(2, 3) OG_A2(4, 5)

#define OG_B4(b) "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
#define OG_B8(b) "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7])
#define OG_B16(b)                                                                            \
  OG_B8(b), "v"(b[8]), "v"(b[9]), "v"(b[10]), "v"(b[11]), "v"(b[12]), "v"(b[13]), "v"(b[14]), \
      "v"(b[15])

// N (8 or 16) steps of R (1 or 2) rows: acc[r] over b[0..N-1] with the
// weights of row r in w[r] (lane u of each row of 16 holds step u's weight).
template <int MODE, int R, int N>
__device__ __forceinline__ void dpp_steps(float (&acc)[R], const float (&w)[R], const float *b) {
  static_assert((R == 1 || R == 2) && (N == 4 || N == 8 || N == 16), "dpp_steps shape");
  if constexpr (MODE == kFast && R == 1 && N == 4)
    asm(OG_FAST1_4 : "+v"(acc[0]) : "v"(w[0]), OG_B4(b));
  else if constexpr (MODE == kFast && R == 1 && N == 8)
    asm(OG_FAST1_8 : "+v"(acc[0]) : "v"(w[0]), OG_B8(b));
  else if constexpr (MODE == kFast && R == 1)
    asm(OG_FAST1_16 : "+v"(acc[0]) : "v"(w[0]), OG_B16(b));
  else if constexpr (MODE == kFast && N == 4)
    asm(OG_FAST2_4 : "+v"(acc[0]), "+v"(acc[1]) : "v"(w[0]), "v"(w[1]), OG_B4(b));
  else if constexpr (MODE == kFast && N == 8)
    asm(OG_FAST2_8 : "+v"(acc[0]), "+v"(acc[1]) : "v"(w[0]), "v"(w[1]), OG_B8(b));
  else if constexpr (MODE == kFast)
    asm(OG_FAST2_16 : "+v"(acc[0]), "+v"(acc[1]) : "v"(w[0]), "v"(w[1]), OG_B16(b));
  else if constexpr (R == 1) {
    float t0, t1;
    if constexpr (N == 4)
      asm(OG_EXACT1_4 : "+v"(acc[0]), "=&v"(t0), "=&v"(t1) : "v"(w[0]), OG_B4(b));
    else if constexpr (N == 8)
      asm(OG_EXACT1_8 : "+v"(acc[0]), "=&v"(t0), "=&v"(t1) : "v"(w[0]), OG_B8(b));
    else
      asm(OG_EXACT1_16 : "+v"(acc[0]), "=&v"(t0), "=&v"(t1) : "v"(w[0]), OG_B16(b));
  } else {
    float t0, t1, t2, t3;
    if constexpr (N == 4)
      asm(OG_EXACT2_4
          : "+v"(acc[0]), "+v"(acc[1]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
          : "v"(w[0]), "v"(w[1]), OG_B4(b));
    else if constexpr (N == 8)
      asm(OG_EXACT2_8
          : "+v"(acc[0]), "+v"(acc[1]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
          : "v"(w[0]), "v"(w[1]), OG_B8(b));
    else
      asm(OG_EXACT2_16
          : "+v"(acc[0]), "+v"(acc[1]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
          : "v"(w[0]), "v"(w[1]), OG_B16(b));
  }
}

// ---------------------------------------------------------------------------
// Chain kernel, for shapes whose outputs are too few to fill the chip and
// whose k is long (the deep layers of a convolution network at batch 1, a
// matrix-vector product, small square products).  There the time is the
// length of one output's chain of k dependent operations, so the waves that
// own outputs ("compute waves") run nothing but that chain: per k step one
// DPP-broadcast fused multiply-add (fast) or multiply then add (exact), the
// B values read from LDS four steps per 16-byte read and the weights one
// read per 16 steps.  A compute wave issues no global load and never waits
// at a barrier for its own LDS reads.  "Producer waves" of the same block
// stream B and a "weight wave" streams the block's weight rows from memory
// into a ring of three LDS stages.
//
// B is read as a stack of "planes": the rows of a row-major matrix (GEMM),
// or the input channels of one (image, group) of a convolution.  A k-chunk
// is CH whole planes, CH*KHW taps in the order (plane, ky, kx).  Producer
// lane groups of BN lanes own CPG planes of a chunk and one column each; a
// lane keeps the byte offset of every one of its taps inside a chunk (its
// column's pixel at each kernel position, or an offset past the buffer for
// a padding tap or a column beyond the tile), so a tap is one buffer load
// with no arithmetic and the padding zeros come from the load itself.  When
// B is a matrix whose rows are 16-byte aligned, a producer lane instead
// loads a 4x4 block (four rows of four columns, 16 bytes each) and stores
// it transposed.  LDS holds a chunk as [tap/4][column][tap%4], so a compute
// lane reads four consecutive taps of its column with one 16-byte read, and
// the weights as [row][tap].
//
// Barriers: iteration t (t = -1 .. chunks-1) ends with one block barrier.
// In iteration t producers store chunk t+2 (t = -1 also stores chunk 0) in
// stage (t+2) % 3, and compute waves read chunk t+1 from stage (t+1) % 3
// into registers while they run the chain of chunk t; they consume those
// reads before the next barrier, so a stage is written two barriers after
// its last read has completed.  Loads past the last chunk reload the last
// chunk (branch-free rings, exact wait counts) and their stores go to a
// stage no one reads again.
// ---------------------------------------------------------------------------
template <int KHW, int BN, int ROWS>
struct ChainShape {
  static constexpr int PG = 4;                         // B producer lane groups
  static constexpr int PW = PG * BN / 64;              // B producer waves
  static constexpr int CPG = KHW == 1 ? 32 : 4;        // planes per group and chunk
  static constexpr int CH = PG * CPG;                  // planes per chunk
  static constexpr int BK = CH * KHW;                  // taps per chunk (128 or 144)
  static constexpr int TPG = CPG * KHW;                // taps per group and chunk
  static constexpr int NW = (ROWS * BK + 63) / 64;     // weight loads per weight-wave lane
  static_assert(PW >= 1 && TPG % 4 == 0 && BK % 16 == 0, "chain chunk shape");
};

// How the chain kernel's producers read B: one tap per load; 4x4 blocks of
// a matrix with 16-byte loads; or, for a 3x3 window with horizontal dilation
// 1, the three taps of a kernel row with one 12-byte load.
// kLdVecT: B given as its transpose (N x K, each column's taps contiguous),
// 16 bytes (4 taps of one column) per load, stored as they are.
enum ChainLoad { kLdTap = 0, kLdVec = 1, kLdRow3 = 2, kLdVecT = 3 };

// Output rows of a chain-kernel block: CW compute waves of (64/BN) lane rows
// and R rows per lane; with the matrix-core compute (MF) a wave's R chains
// are 4 rows each.
constexpr int chain_rows(int CW, int BN, int R, bool MF) { return MF ? CW * 4 * R : CW * (64 / BN) * R; }

template <int MODE, bool CONV, int LD, int KH, int KW, int BN, int CW, int R, bool MF>
__global__ void __launch_bounds__(64 * (CW + ChainShape<KH * KW, BN, chain_rows(CW, BN, R, MF)>::PW + 1))
    chain_kernel(Problem p) {
  constexpr bool VEC = LD == kLdVec, ROW3 = LD == kLdRow3, VT = LD == kLdVecT;
  constexpr int KHW = KH * KW;
  constexpr int RW = 64 / BN;                    // lane rows of a compute wave
  constexpr int ROWS = chain_rows(CW, BN, R, MF);  // output rows of a block
  static_assert(!MF || (BN == 64 && MODE == kFast), "matrix-core chains: 64 columns, fast mode");
  using CS = ChainShape<KHW, BN, ROWS>;
  constexpr int BK = CS::BK, NQ = BK / 4, NB = BK / 16;
  constexpr int TPG = CS::TPG, CPG = CS::CPG, CH = CS::CH, PW = CS::PW, NW = CS::NW;
  constexpr int NWV = (ROWS * BK / 4 + 63) / 64;  // 16-byte weight loads per weight-wave lane
  constexpr int NWM = NW > 4 * NWV ? NW : 4 * NWV;  // weight-wave registers per chunk
  constexpr int NS = 3, DP = 2, DW = NWM > 20 ? 2 : 4, U = 4;  // LDS stages, ring depths, unroll
  // compute: register blocks of 16 taps, read-ahead, unroll (in chunks)
  constexpr int RB = MF ? 3 : 4, LA = RB - 1, UC = MF ? 3 : 4;
  constexpr int NBL = VEC || VT ? BK / 64 : 0;  // 4x4 blocks per producer lane (16-byte loads)
  static_assert(U % DP == 0 && U % DW == 0 && (UC * NB) % RB == 0, "unroll");
  static_assert(!(VEC || VT) || (!CONV && KHW == 1 && BK % 64 == 0),
                "16-byte producer loads: matrix B only");
  static_assert(!ROW3 || (CONV && KH == 3 && KW == 3), "row loads: 3x3 windows only");
  __shared__ __align__(16) float4 stage[NS][NQ * BN];
  __shared__ __align__(16) float wstage[NS][ROWS * BK];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cl = lane % BN;

  // the tile's columns: matrix columns, or output pixels of one image
  int img = 0, cbase;
  if (CONV) {
    const int tpi = (p.OHW + BN - 1) / BN;
    img = tc.tn / tpi;
    cbase = (tc.tn - img * tpi) * BN;
  } else {
    cbase = tc.tn * BN;
  }
  const int ncols = CONV ? p.OHW : p.N;
  const int cidx = cbase + cl;
  const bool col_ok = cidx < ncols;

  const float *pbase = CONV ? p.B + img * p.x_img + tc.g * p.x_grp : p.B;
  const int64_t pstride = CONV ? (int64_t)p.HW : p.ldb;
  const int pcount = CONV ? p.K / KHW : p.K;
  const int nchunks = (pcount + CH - 1) / CH;
  const int last = nchunks - 1;
  const int row0 = tc.tm * ROWS;  // first row of the block
  const int mlast = p.M - 1;
  if (nchunks == 0 && wave >= CW) return;  // k = 0: no barrier is ever reached

  if (wave == CW + PW) {
    // ---------------- weight wave: the block's rows, [row][tap] ----------------
    // With aligned rows (p.a_vec, uniform) each lane loads 16 bytes (4 taps)
    // per load, NWV loads per chunk; else one tap per load, NW loads.
    const float *wbase = p.A + tc.g * p.a_gstride + (int64_t)min(row0, mlast) * p.lda;
    const bool wv = p.a_vec != 0;
    // byte offset of load i of this lane inside a chunk (past the buffer when
    // the load is beyond the block's rows or beyond k): tap-wise, element idx
    // of [row][tap]; 16-byte, quad idx of [row][tap/4]
    auto woffset = [&](int i, int k0, auto vec) __attribute__((always_inline)) -> uint32_t {
      constexpr bool V = decltype(vec)::value;
      constexpr int per = V ? BK / 4 : BK, width = V ? 4 : 1, lim = V ? ROWS * BK / 4 : ROWS * BK;
      const int idx = i * 64 + lane;
      const int r = idx / per, t = (idx - r * per) * width;
      if (idx >= lim || k0 + t >= p.K) return kOutside;
      return (uint32_t)((int64_t)(min(row0 + r, mlast) - min(row0, mlast)) * p.lda * 4 + 4 * t);
    };
    float rw[DW][NWM];
    auto load = [&](int c, auto slot) __attribute__((always_inline)) {
      constexpr int S = decltype(slot)::value;
      const int k0 = c * BK;
      const __amdgpu_buffer_rsrc_t rs = buffer_at(wbase + k0, kRange);
      if (wv) {
#pragma unroll
        for (int i = 0; i < NWV; ++i)
          load4(rs, woffset(i, k0, std::true_type{}), &rw[S][4 * i]);
      } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) rw[S][i] = load1(rs, woffset(i, k0, std::false_type{}));
      }
    };
    // chunk c into stage st; in fast mode, in a chunk that runs past K, the
    // weights of taps at or beyond K are then overwritten with -0 (B's are
    // +0), so each padded term adds a product of -0 (the lane's own stores:
    // no barrier between; with 16-byte loads K is a multiple of 4, so a quad
    // is wholly past or not)
    auto store = [&](auto slot, int st, int c) __attribute__((always_inline)) {
      constexpr int S = decltype(slot)::value;
      if (wv) {
#pragma unroll
        for (int i = 0; i < NWV; ++i)
          if (i * 64 + lane < ROWS * BK / 4)
            *reinterpret_cast<float4 *>(&wstage[st][4 * (i * 64 + lane)]) =
                make_float4(rw[S][4 * i], rw[S][4 * i + 1], rw[S][4 * i + 2], rw[S][4 * i + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < NW; ++i)
          if (i * 64 + lane < ROWS * BK) wstage[st][i * 64 + lane] = rw[S][i];
      }
      const int k0 = c * BK;
      if (MODE == kFast && k0 + BK > p.K) {
        if (wv) {
          for (int idx = lane; idx < ROWS * BK / 4; idx += 64)
            if (k0 + 4 * (idx % (BK / 4)) >= p.K)
              *reinterpret_cast<float4 *>(&wstage[st][4 * idx]) = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
        } else {
          for (int idx = lane; idx < ROWS * BK; idx += 64)
            if (k0 + idx % BK >= p.K) wstage[st][idx] = -0.0f;
        }
      }
    };
    static_for<DW>([&](auto j) __attribute__((always_inline)) { load(min((int)decltype(j)::value, last), j); });
    store(std::integral_constant<int, 0>{}, 0, 0);
    load(min(DW, last), std::integral_constant<int, 0>{});
    for (int t0 = -1; t0 < nchunks; t0 += U) {
      static_for<U>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        const int t = t0 + J;
        if (t < nchunks) {
          const int v = t + 2;  // the chunk stored now (slot (J + 1) % DW holds it)
          store(std::integral_constant<int, (J + 1) % DW>{}, v % NS, v);
          load(min(v + DW, last), std::integral_constant<int, (J + 1) % DW>{});
          __syncthreads();
        }
      });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  if (wave >= CW) {
    // ---------------- B producers ----------------
    const int pw = wave - CW;
    constexpr int NL = VEC || VT ? 4 * NBL : ROW3 ? TPG / 3 : TPG;  // loads per lane and chunk
    uint32_t off[NL];
    int qv[VT ? NL : 1];  // transposed B: the tap quad of each load
    int grp = 0, qb[VEC ? NBL : 1], cb[VEC ? NBL : 1];
    // row loads: the load of kernel row ky starts at column s0 of the input
    // row, s0 = clamp(ix0, 0, W-3); tap kx is component kx + d (d = ix0 - s0,
    // -1, 0 or 1 with left and right pads <= 1) when its column is inside
    bool kin[3] = {false, false, false};
    int dsh = 0;
    if constexpr (VEC) {
      // lane -> 4x4 blocks: taps 4qb..4qb+3 of columns 4cb..4cb+3
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        const int id = i * 64 * PW + pw * 64 + lane;
        qb[i] = id / (BN / 4);
        cb[i] = id - qb[i] * (BN / 4);
        const bool ok = cbase + 4 * cb[i] < ncols;  // ncols is a multiple of 4 here
#pragma unroll
        for (int j = 0; j < 4; ++j)
          off[4 * i + j] =
              ok ? (uint32_t)(((int64_t)(4 * qb[i] + j) * pstride + cbase + 4 * cb[i]) * 4) : kOutside;
      }
    } else if constexpr (VT) {
      // lane -> (column, tap quad) pairs, columns fastest: a load instruction
      // reads 16 bytes of each of BN columns (rows of the N x K operand),
      // and a wave's LDS stores are contiguous.  Offsets are from column
      // cbase of the chunk's first tap.
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int id = j * 64 * PW + pw * 64 + lane;
        const int col = id % BN;
        qv[j] = id / BN;
        off[j] = cbase + col < ncols ? (uint32_t)(((int64_t)col * pstride + 4 * qv[j]) * 4) : kOutside;
      }
    } else if constexpr (ROW3) {
      grp = pw * (64 / BN) + lane / BN;
      const int oy = col_ok ? cidx / p.OW : 0;
      const int ox = col_ok ? cidx - oy * p.OW : 0;
      const int iy0 = oy * p.sH - p.pT, ix0 = ox * p.sW - p.pL;
      const int s0 = min(max(ix0, 0), p.W - 3);
      dsh = ix0 - s0;
#pragma unroll
      for (int kx = 0; kx < 3; ++kx) kin[kx] = col_ok && (unsigned)(ix0 + kx) < (unsigned)p.W;
      uint32_t roff[3];
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const int iy = iy0 + ky * p.dH;
        roff[ky] = col_ok && (unsigned)iy < (unsigned)p.H ? (uint32_t)(4 * (iy * p.W + s0)) : kOutside;
      }
#pragma unroll
      for (int j = 0; j < CPG; ++j)
#pragma unroll
        for (int ky = 0; ky < 3; ++ky) {
          const int64_t o = (int64_t)(grp * CPG + j) * pstride * 4 + roff[ky];
          off[j * 3 + ky] = (roff[ky] == kOutside || o >= (int64_t)kOutside) ? kOutside : (uint32_t)o;
        }
    } else {
      grp = pw * (64 / BN) + lane / BN;
      uint32_t voff[KHW];
      if (CONV) {
        const int oy = col_ok ? cidx / p.OW : 0;
        const int ox = col_ok ? cidx - oy * p.OW : 0;
        const int iy0 = oy * p.sH - p.pT, ix0 = ox * p.sW - p.pL;
#pragma unroll
        for (int ky = 0; ky < KH; ++ky)
#pragma unroll
          for (int kx = 0; kx < KW; ++kx) {
            const int iy = iy0 + ky * p.dH, ix = ix0 + kx * p.dW;
            const bool in = col_ok && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
            voff[ky * KW + kx] = in ? (uint32_t)(4 * (iy * p.W + ix)) : kOutside;
          }
      } else {
        voff[0] = col_ok ? (uint32_t)(4 * cidx) : kOutside;
      }
#pragma unroll
      for (int j = 0; j < CPG; ++j)
#pragma unroll
        for (int t = 0; t < KHW; ++t) {
          const int64_t o = (int64_t)(grp * CPG + j) * pstride * 4 + voff[t];
          off[j * KHW + t] = (voff[t] == kOutside || o >= (int64_t)kOutside) ? kOutside : (uint32_t)o;
        }
    }
    float rb[DP][VEC || VT ? 16 * NBL : TPG];
    auto load = [&](int c, auto slot) __attribute__((always_inline)) {
      constexpr int S = decltype(slot)::value;
      if constexpr (VT) {
        // k is a multiple of 4 here: a tap quad is wholly inside or past k
        const __amdgpu_buffer_rsrc_t rt =
            buffer_at(pbase + (int64_t)cbase * pstride + (int64_t)c * CH, kRange);
        const int kleft = pcount - c * CH;
#pragma unroll
        for (int j = 0; j < NL; ++j) load4(rt, 4 * qv[j] < kleft ? off[j] : kOutside, &rb[S][4 * j]);
        return;
      }
      const int valid = min(max(pcount - c * CH, 0), CH);  // planes of the chunk that exist
      // (the range is uniform; readfirstlane keeps the descriptor in scalar
      // registers where the compiler would otherwise clamp it on the VALU)
      const uint32_t range =
          __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)valid * pstride * 4));
      const __amdgpu_buffer_rsrc_t rs = buffer_at(pbase + (int64_t)c * CH * pstride, range);
      if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < 4 * NBL; ++j) load4(rs, off[j], &rb[S][4 * j]);
      } else if constexpr (ROW3) {
#pragma unroll
        for (int e = 0; e < TPG / 3; ++e) load3(rs, off[e], &rb[S][3 * e]);
      } else {
#pragma unroll
        for (int e = 0; e < TPG; ++e) rb[S][e] = load1(rs, off[e]);
      }
    };
    auto store = [&](auto slot, int st) __attribute__((always_inline)) {
      constexpr int S = decltype(slot)::value;
      if constexpr (VT) {
        // load j holds taps 4 qv[j] .. + 3 of column (lane-order) j: already
        // the [tap/4][column] layout
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int id = j * 64 * PW + pw * 64 + lane;
          stage[st][qv[j] * BN + id % BN] =
              make_float4(rb[S][4 * j], rb[S][4 * j + 1], rb[S][4 * j + 2], rb[S][4 * j + 3]);
        }
        return;
      }
      if constexpr (VEC) {
        // rb[16i + 4j + jj] is (tap 4qb + j, column 4cb + jj) of block i:
        // store each column's four taps
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          float4 *dst = stage[st] + qb[i] * BN + 4 * cb[i];
          const float *v = &rb[S][16 * i];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) dst[jj] = make_float4(v[jj], v[4 + jj], v[8 + jj], v[12 + jj]);
        }
      } else {
        if constexpr (ROW3) {
          // the loaded row segments -> the three taps of each kernel row
#pragma unroll
          for (int e = 0; e < TPG / 3; ++e) {
            const float c0 = rb[S][3 * e], c1 = rb[S][3 * e + 1], c2 = rb[S][3 * e + 2];
            rb[S][3 * e] = kin[0] ? (dsh > 0 ? c1 : c0) : 0.0f;
            rb[S][3 * e + 1] = kin[1] ? (dsh < 0 ? c0 : dsh > 0 ? c2 : c1) : 0.0f;
            rb[S][3 * e + 2] = kin[2] ? (dsh < 0 ? c1 : c2) : 0.0f;
          }
        }
        float4 *dst = stage[st] + grp * (TPG / 4) * BN + cl;
#pragma unroll
        for (int q = 0; q < TPG / 4; ++q)
          dst[q * BN] = make_float4(rb[S][4 * q], rb[S][4 * q + 1], rb[S][4 * q + 2], rb[S][4 * q + 3]);
      }
    };
    static_for<DP>([&](auto j) __attribute__((always_inline)) { load(min((int)decltype(j)::value, last), j); });
    store(std::integral_constant<int, 0>{}, 0);
    load(min(DP, last), std::integral_constant<int, 0>{});
    for (int t0 = -1; t0 < nchunks; t0 += U) {
      static_for<U>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        const int t = t0 + J;
        if (t < nchunks) {
          const int v = t + 2;  // the chunk stored now (slot (J + 1) % DP holds it)
          store(std::integral_constant<int, (J + 1) % DP>{}, v % NS);
          load(min(v + DP, last), std::integral_constant<int, (J + 1) % DP>{});
          __syncthreads();
        }
      });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // ---------------- compute ----------------
  // The chain runs in blocks of 16 taps; block L of the run (chunk L / NB,
  // block L % NB of it) sits in register slot L % RB, read from LDS LA
  // blocks before it is used.
  //
  // DPP form: lane l owns column l % BN of lane row l / BN, R rows per lane;
  // the weight register holds 16 taps of a row, one per lane of a row of 16.
  // Matrix-core form (MF): each of the wave's R chains is 4 rows x 64
  // columns in one v_mfma_f32_4x4x1_16b_f32 per k: its 16 blocks of 4x4
  // share the 4 rows; lane l gives the B value of column l and holds the 4
  // rows of column l (register i = row i).  The weights come through the
  // instruction's A broadcast (cbsz 4: every block takes the A values of
  // block abid): one register holds 16 taps of the chain's 4 rows, lane
  // 4b + i the weight of row i at tap b, and step u of the 16 broadcasts
  // block u.  Each output element of the instruction is one fused
  // multiply-add, so a chain over increasing k is fast mode (the only mode
  // this form runs).
  const int lr = lane / BN;                 // lane row of the wave (DPP form)
  const int rb0 = MF ? wave * 4 * R : wave * RW * R + lr * R;  // first row of the lane / wave
  float4 bq[RB][4];
  float wq[RB][MF ? 1 : R];
  float wa[RB][MF ? R : 1];
  auto read = [&](auto slot, int st, auto blk) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value, B = decltype(blk)::value;
    const float4 *src = stage[st] + 4 * B * BN + cl;
#pragma unroll
    for (int i = 0; i < 4; ++i) bq[S][i] = src[i * BN];
    if constexpr (MF) {
#pragma unroll
      for (int c = 0; c < R; ++c) wa[S][c] = wstage[st][(rb0 + 4 * c + (lane & 3)) * BK + 16 * B + (lane >> 2)];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) wq[S][r] = wstage[st][(rb0 + r) * BK + 16 * B + (lane & 15)];
    }
  };
  float acc[R];
  f32x4 acc4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0f;
    acc4[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  if (nchunks > 0) {
    // The compute waves write no LDS, so their barrier needs no fence and no
    // wait for their own reads (the asm's memory clobber keeps the compiler
    // from moving LDS reads across it).  Reads never run more than a chunk
    // ahead, so they only touch stages complete at the previous barrier.
    asm volatile("s_barrier" ::: "memory");
    static_for<LA>([&](auto l) __attribute__((always_inline)) {
      constexpr int L = decltype(l)::value;
      read(std::integral_constant<int, L % RB>{}, 0, std::integral_constant<int, L % NB>{});
    });
    for (int t0 = 0; t0 < nchunks; t0 += UC) {
      static_for<UC>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        const int t = t0 + J;
        if (t < nchunks) {
          static_for<NB>([&](auto bb) __attribute__((always_inline)) {
            constexpr int L = J * NB + decltype(bb)::value;  // block of the unrolled run
            constexpr int LN = L + LA;                        // the block read now
            read(std::integral_constant<int, LN % RB>{}, (t0 + LN / NB) % NS,
                 std::integral_constant<int, LN % NB>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MF) {
              static_for<16>([&](auto uq) __attribute__((always_inline)) {
                constexpr int u = decltype(uq)::value;
#pragma unroll
                for (int c = 0; c < R; ++c) {
                  acc4[c] = __builtin_amdgcn_mfma_f32_4x4x1f32(wa[L % RB][c], bq[L % RB][u / 4][u % 4],
                                                                acc4[c], 4, u, 0);
                }
              });
            } else {
              float b[16];
#pragma unroll
              for (int u = 0; u < 16; ++u) b[u] = bq[L % RB][u / 4][u % 4];
              float w[R];
#pragma unroll
              for (int r = 0; r < R; ++r) w[r] = wq[L % RB][r];
              dpp_steps<MODE, R, 16>(acc, w, b);
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_barrier" ::: "memory");
        }
      });
    }
  }
  // One uniform test picks the store loop with or without the epilogue.
  auto store_all = [&](auto epi) __attribute__((always_inline)) {
    constexpr bool E = decltype(epi)::value;
    if constexpr (MF) {
      if (col_ok) {
        float *base = out_ptr<CONV ? kBGather : kBMatrix>(p, tc.g, 0, CONV ? img * p.OHW + cidx : cidx);
        const int64_t rstride = CONV ? (int64_t)p.OHW : p.ldc;
        float pb[R][4], pr[R][4];
        if constexpr (E) {
#pragma unroll
          for (int c = 0; c < R; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = row0 + rb0 + 4 * c + i;
              pb[c][i] = epi_bias(p, row < p.M, tc.g * p.M + row);
              pr[c][i] = epi_res(p, row < p.M, base + (int64_t)(row < p.M ? row : 0) * rstride);
            }
        }
#pragma unroll
        for (int c = 0; c < R; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = row0 + rb0 + 4 * c + i;
            if (row < p.M) {
              if constexpr (E)
                base[(int64_t)row * rstride] = finish_with(p, acc4[c][i], pb[c][i], pr[c][i]);
              else
                base[(int64_t)row * rstride] = finish<false>(p, acc4[c][i], 0, base);
            }
          }
      }
      return;
    }
    if (col_ok) {
      float *base = out_ptr<CONV ? kBGather : kBMatrix>(p, tc.g, 0, CONV ? img * p.OHW + cidx : cidx);
      const int64_t rstride = CONV ? (int64_t)p.OHW : p.ldc;
      float pb[R], pr[R];
      if constexpr (E) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = row0 + rb0 + r;
          pb[r] = epi_bias(p, row < p.M, tc.g * p.M + row);
          pr[r] = epi_res(p, row < p.M, base + (int64_t)(row < p.M ? row : 0) * rstride);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + rb0 + r;
        if (row < p.M) {
          if constexpr (E)
            base[(int64_t)row * rstride] = finish_with(p, acc[r], pb[r], pr[r]);
          else
            base[(int64_t)row * rstride] = finish<false>(p, acc[r], 0, base);
        }
      }
    }
  };
  if (p.bias == nullptr && p.res == nullptr && p.act == 0)
    store_all(std::false_type{});
  else
    store_all(std::true_type{});
}

// ---------------------------------------------------------------------------
// Halo kernel: fast-mode KH x KW convolutions on the matrix cores, for
// layers whose outputs split into enough chains of 4 output channels to fill
// the chip (a batch of images through the middle of a convolution network).
//
// A block is CW waves over 64 lanes of one image; wave w owns R chains of 4
// output channels.  Per tap a chain is one v_mfma_f32_4x4x1_16b_f32: its 16
// blocks of 4x4 share the 4 rows, lane l gives the input value of its
// pixel's window at that tap and holds the 4 outputs of its pixel (register
// i = output channel i of the chain), each a single fused multiply-add -- so
// a chain over increasing k is the fast mode's ordered sum.  The weights come
// through the instruction's A broadcast (cbsz 4: every block takes the A
// values of block abid): one register holds 16 taps of the chain's 4 rows,
// lane 4b + i the weight of row i at tap b, and tap u of the 16 broadcasts
// block u.  The rows are the wave's own: it streams them straight from
// memory into its own ring of NWS LDS stages, NWS-1 chunks ahead, and reads
// them into registers before the chunk's last quad (every lane of every load
// has a place in the stage, so the loads are unconditional and the waits
// count them exactly).
//
// Lanes and pixels: at stride 1 (p.vpitch = W + pL + pR, the padded row)
// the 64 lanes take 64 consecutive cells of the output rows laid out as
// wide as the padded input row, the last pL + pR cells of each row being no
// pixel (computed, not stored), so the 64 lanes' reads of a tap are 64
// consecutive cells of the stage; otherwise (p.vpitch = 0) they take 64
// consecutive output pixels.
//
// The input is staged per chunk of CC = 16 channels (CC*KHW taps in the
// order channel, kernel row, kernel column).  The block stages the halo of
// its lanes' windows with the padding in place: the rows they reach, each
// as wide as the padded input row, the padding cells +0 (written once,
// before the first chunk) and the input's rows -- contiguous in x, read with
// 4-byte (HV: 16-byte) loads, wave w loading channels w*CPW.. -- stored in
// the middle.  LDS holds a chunk as [cell][channel]: a cell is the CC
// channels of one input position and 4 floats of padding (80 bytes, so 8
// lanes reading 16 bytes of 8 consecutive cells meet 8 different groups of
// banks).  A window position is then always a cell at a fixed distance from
// the lane's first cell of its kernel row, and one 16-byte read brings 4
// channels of one tap position: with the kernel row's pointer, the kernel
// column and the channel quad sit in the read's immediate offset (no
// address arithmetic per tap).  Taps run in k order: quad q of a chunk is
// its channels 4q..4q+3, each over the KHW window positions, read as KHW
// 16-byte reads (one per position) and run as 4*KHW chain steps.  A wave
// stores its CPW channels of an input position as one 16-byte (CPW = 2:
// 8-byte) write.  Lanes past the input's part of the halo write a spare cell
// past the rows.  Channels past the group's last are staged as +0 (their
// loads are out of range) and their weights are made -0, so those taps add a
// product of -0 (fast mode's padding).
//
// The staging never stops the matrix cores: chunk c's products run in two
// halves, and between them each wave stores its part of chunk c+1's halo
// (loaded during chunk c-1) into the next of three LDS buffers, issues the
// loads of chunk c+2 and meets the others at the chunk's one barrier; the
// second half then reads chunk c+1's first quad while it runs.  Buffer
// (c+1) % 3 was last read in chunk c-2, which every wave finished before the
// barrier of chunk c-1.  With two buffers (NBUF = 2, for halos whose three
// buffers would not leave LDS for as many blocks per compute unit) the store
// waits for that barrier, and a second barrier before the chunk's last quad
// makes chunk c+1's halo visible to the reads of its first.  p.hrows: rows a
// tile stages at most (with its padding rows); a buffer is
// hrows * (W + pL + pR) + 3 cells (two cells read past the rows by lanes of
// no pixel, one spare written by idle lanes).
// ---------------------------------------------------------------------------
template <int MODE, int KH, int KW, int R, int CW, int NI, bool HV, bool AV, int NWS, int NBUF, bool DPP>
__global__ void __launch_bounds__(64 * CW) halo_kernel(Problem p) {
  constexpr int KHW = KH * KW;
  constexpr int CC = 16;                 // channels per chunk
  constexpr int BK = CC * KHW;           // taps per chunk
  constexpr int NG = BK / 16;            // 16-tap weight groups per chunk
  constexpr int NQC = CC / 4;            // channel quads per chunk
  constexpr int QT = 4 * KHW;            // taps per quad
  constexpr int CSTR = CC + 4;           // floats of a staged cell
  constexpr int C4 = CSTR / 4;           // its 16-byte units
  constexpr int CPW = CC / CW;           // channels each wave stages
  constexpr int VW = HV ? 4 : 1;         // floats per halo load
  constexpr int RA = DPP ? 1 : 4;                 // rows per chain: a lane's own (DPP), 4 (matrix cores)
  constexpr int WROWS = RA * R, WST = WROWS * BK;  // a wave's weight rows; floats of a weight stage
  constexpr int WW = AV ? 4 : 1;                  // taps per weight load
  constexpr int NQW = WST / WW, NIW = (NQW + 63) / 64;  // weight loads per stage, per lane
  constexpr int WSTP = NIW * 64 * WW;             // floats of a stage, every lane's place included
  constexpr int NL = CPW * NI;                    // halo loads per chunk, per lane
  static_assert(BK % 16 == 0 && (CPW == 4 || CPW == 2) && NQC % 2 == 0, "halo chunk shape");
  static_assert(NWS == 2 || NWS == 3, "two or three weight stages per wave");
  static_assert(NBUF == 2 || NBUF == 3, "two or three halo buffers");
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  // [NBUF][cells][CSTR] halo, then per wave [NWS][WSTP] weights
  extern __shared__ __align__(16) float hs[];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the lanes' cells: rows of vw cells, of which the first OW are pixels
  const int vw = p.vpitch > 0 ? p.vpitch : p.OW;
  const int ncell = p.OHW / p.OW * vw;  // cells of an image
  const int tpi = (ncell + 63) / 64;    // tiles per image
  const int img = tc.tn / tpi;
  const int pbase = (tc.tn - img * tpi) * 64;
  const int cell = pbase + lane;
  const int cy = cell / vw, cx = cell - cy * vw;
  const bool valid = cell < ncell && cx < p.OW;
  const int pix = cy * p.OW + cx;  // the lane's output pixel, where valid
  const int cin_g = p.K / KHW;
  const int wp = p.W + p.pL + p.pR;       // a staged row: the padded input row
  const int spare = p.hrows * wp + 2;     // the cell idle lanes write
  const int bufsz = (spare + 1) * CSTR;   // floats of a buffer
  // the tile's staged rows: input rows ybase .. (padding rows included), of
  // which r0 .. r1 are the input's
  const int oy_first = pbase / vw, oy_last = min(pbase + 63, ncell - 1) / vw;
  const int ybase = oy_first * p.sH - p.pT;
  const int r0 = max(ybase, 0);
  const int r1 = min(oy_last * p.sH - p.pT + (KH - 1) * p.dH, p.H - 1);
  // input floats of a channel (none when every window of the tile lies in
  // the padding rows)
  const int hlen = max(r1 - r0 + 1, 0) * p.W;

  // this lane's first cell of each kernel row, in the buffer of the chunk
  // being run, and in the next chunk's
  const f32x4 *tp[KH], *tn[KH];
  {
    // (lanes of no pixel read the cells of their own place in the rows: at
    // stride 1, within hrows rows of the stage plus two cells, which only
    // they read; past an image's last row, the first pixel's cells)
    const bool in_rows = cell < ncell || p.vpitch > 0;
    const int oy = in_rows ? cy : oy_first;
    const int ox = in_rows ? cx : 0;
    const f32x4 *hs4 = reinterpret_cast<const f32x4 *>(hs);
#pragma unroll
    for (int ky = 0; ky < KH; ++ky)
      tp[ky] = hs4 + (((oy - oy_first) * p.sH + ky * p.dH) * wp + ox * p.sW) * C4;
  }
  // the cell each halo element of this lane goes to (the same in every
  // chunk; the spare cell for lanes past the halo)
  int hcell[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = VW * (lane + 64 * i), rr = q / p.W;
    hcell[i] = q < hlen ? (r0 - ybase + rr) * wp + p.pL + q - rr * p.W : spare;
  }
  // +0 everywhere (the padding cells keep it), before the first stores
  for (int e = threadIdx.x; e < NBUF * bufsz / 4; e += 64 * CW)
    reinterpret_cast<f32x4 *>(hs)[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // this wave's weight rows, streamed by the wave itself into its own pair
  // of LDS stages ([row][tap], WW taps per lane and load, straight from
  // memory into LDS) one chunk ahead; read back per chunk, lane 4b + i
  // taking row i of each chain at tap b of each 16-tap group
  const int wrow0 = tc.tm * (WROWS * CW) + wave * WROWS;  // first row of the wave
  const int wbase = min(wrow0, p.M - 1);
  const __amdgpu_buffer_rsrc_t wrs =
      buffer_at(p.A + tc.g * p.a_gstride + (int64_t)wbase * p.lda, kRange);
  float *const wring = hs + NBUF * bufsz + wave * NWS * WSTP;
  uint32_t wq[NIW];  // byte offset of the lane's taps of load n in chunk 0, or kOutside
  int wt[NIW];       // their first tap in a chunk
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int q = n * 64 + lane, r = q / (BK / WW);
    wt[n] = (q - r * (BK / WW)) * WW;
    wq[n] = q < NQW && wrow0 + r < p.M
                ? (uint32_t)((int64_t)(wrow0 + r - wbase) * p.lda * 4 + 4 * wt[n])
                : kOutside;
  }
  const int tb = lane >> 2;  // the lane's tap within a 16-tap group

  const float *xg = p.B + img * p.x_img + tc.g * p.x_grp + (int64_t)r0 * p.W;  // row r0 of channel 0
  const int nch = (cin_g + CC - 1) / CC, last = nch - 1;
  float rb[2][CPW][NI * VW];  // halo of chunk c in slot c % 2
  // weights of chunk c (read from its stage) in slot c % 2: matrix cores,
  // 16-tap groups of the chunk; DPP, per quad its runs of 16, 16 and 4 taps
  constexpr int NGW = DPP ? 3 * NQC : NG;
  static_assert(!DPP || QT == 36, "DPP runs of a quad: 16, 16, 4 taps");
  float wv[2][R][NGW];
  f32x4 qb[2][KHW];           // a quad's input values (4 channels per position), read one quad ahead
  f32x4 acc[R];   // matrix cores: the 4 rows of chain r at the lane's pixel
  float accd[R];  // DPP: row r at the lane's pixel
#pragma unroll
  for (int c = 0; c < R; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, accd[c] = 0.0f;

  auto load_halo = [&](int c, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    c = min(c, last);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int ch = c * CC + wave * CPW + j;  // wave-uniform
      // a channel past the group's last gets an empty range: +0
      const __amdgpu_buffer_rsrc_t rs = buffer_at(xg + (int64_t)min(ch, cin_g - 1) * p.HW,
                                                  ch < cin_g ? (uint32_t)(4 * hlen) : 0u);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t off = (uint32_t)(4 * VW * (lane + 64 * i));
        if constexpr (HV)
          load4(rs, off, &rb[S][j][4 * i]);
        else
          rb[S][j][i] = load1(rs, off);
      }
    }
  };
  // chunk c's weights into stage c % NWS (loads past the last chunk reload it)
  auto load_w = [&](int c) __attribute__((always_inline)) {
    const int k0 = min(c, last) * BK;
    float *dst = wring + (c % NWS) * WSTP;
#pragma unroll
    for (int n = 0; n < NIW; ++n) {
      const uint32_t off = wq[n] != kOutside && k0 + wt[n] < p.K ? wq[n] + 4 * k0 : kOutside;
      auto *to = (__attribute__((address_space(3))) void *)(dst + n * 64 * WW);
      if constexpr (AV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, to, 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, to, 4, off, 0, 0, 0);
    }
  };
  // chunk c's weights from its stage into slot S, once its loads are in:
  // after them the wave has issued exactly `later` loads (a chunk's halo
  // and weight loads go out in a fixed order)
  auto read_w = [&](int c, auto slot, auto later) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value, LATER = decltype(later)::value;
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(LATER < 63 ? LATER : 63) : "memory");
    float *stg = wring + (c % NWS) * WSTP;
    // in a chunk running past k (the last one at most) the taps past k get
    // -0 weights, written over the wave's own stage (its LDS operations run
    // in order)
    if ((c + 1) * BK > p.K) {
      for (int e = lane; e < WST; e += 64)
        if (c * BK + e % BK >= p.K) stg[e] = -0.0f;
    }
    if constexpr (DPP) {
      // lane u of each row of 16 holds tap u of the run (for row_newbcast);
      // a quad's third run has 4 taps (lanes past them read taps of the next
      // quad or the stage's padding, unused)
      const float *src = stg + (lane & 15);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < NQC; ++q)
#pragma unroll
          for (int j = 0; j < 3; ++j) wv[S][r][3 * q + j] = src[r * BK + QT * q + 16 * j];
    } else {
      const float *src = stg + (lane & 3) * BK + tb;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) wv[S][r][gi] = src[4 * r * BK + 16 * gi];
    }
  };
  // the wave's CPW channels of each of its halo elements, one write per
  // input position
  auto store_halo = [&](auto slot, int buf) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    float *dst = hs + buf * bufsz + wave * CPW;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        // (16-byte loads: W is a multiple of 4, so the four are in one row)
        const int at = (hcell[i] + (hcell[i] == spare ? 0 : e)) * CSTR;
        if constexpr (CPW == 4)
          *reinterpret_cast<f32x4 *>(dst + at) =
              f32x4{rb[S][0][VW * i + e], rb[S][1][VW * i + e], rb[S][2][VW * i + e], rb[S][3][VW * i + e]};
        else
          *reinterpret_cast<f32x2 *>(dst + at) = f32x2{rb[S][0][VW * i + e], rb[S][1][VW * i + e]};
      }
  };
  // quad Q of a chunk (4 channels at each window position) through the
  // kernel-row pointers ptr into qb[B]
  auto read = [&](auto quad, auto into, const f32x4 *(&ptr)[KH]) __attribute__((always_inline)) {
    constexpr int Q = decltype(quad)::value, B = decltype(into)::value;
    static_for<KHW>([&](auto pq) __attribute__((always_inline)) {
      constexpr int pos = decltype(pq)::value, ky = pos / KW, kx = pos % KW;
      qb[B][pos] = ptr[ky][kx * C4 + Q];
    });
  };
  // the products of quad Q of chunk c (weights in slot S, inputs in qb[B]):
  // its taps in k order, channel 4Q + ci at window position pos.  Fast
  // mode: the chain step itself, one fused multiply-add per output.  Exact
  // mode: the matrix core forms the rounded products (C = +0: fma(w, x, +0)
  // is round(w * x), but +0 for an exact -0 product, which cannot change a
  // sum that is never -0) and separately rounded adds take them into the
  // sums in k order, two taps at a time, the products of the next two taps
  // issued before the adds of these.  Empty asm statements order the steps
  // (an input passes through one before its products, the sums through one
  // after their adds): the products do not depend on the sums, and the
  // compiler would otherwise issue every product of the quad first and run
  // out of registers.
  auto products = [&](auto quad, auto slot, auto from) __attribute__((always_inline)) {
    constexpr int Q = decltype(quad)::value, S = decltype(slot)::value, B = decltype(from)::value;
    if constexpr (DPP) {
      // runs of 16, 16 and 4 taps, each one asm block of DPP steps (weights
      // broadcast from lane u of the run; exact mode's products and sums
      // interleaved inside the block)
      static_for<3>([&](auto jq) __attribute__((always_inline)) {
        constexpr int j = decltype(jq)::value, n = j < 2 ? 16 : 4;
        float b[n];
        static_for<n>([&](auto uq) __attribute__((always_inline)) {
          constexpr int t = 16 * j + decltype(uq)::value, ci = t / KHW, pos = t % KHW;
          b[decltype(uq)::value] = qb[B][pos][ci];
        });
        float w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = wv[S][r][3 * Q + j];
        dpp_steps<MODE, R, n>(accd, w, b);
      });
    } else if constexpr (MODE == kFast) {
      static_for<QT>([&](auto tq) __attribute__((always_inline)) {
        constexpr int t = decltype(tq)::value, s = QT * Q + t, ci = t / KHW, pos = t % KHW;
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[r] = __builtin_amdgcn_mfma_f32_4x4x1f32(wv[S][r][s / 16], qb[B][pos][ci], acc[r], 4, s % 16, 0);
      });
    } else {
      static_assert(QT % 2 == 0, "exact steps go in pairs of taps");
      constexpr int NP = QT / 2;
      f32x4 pr[2][2][R];  // the products of a pair of taps, by the pair's parity
      auto issue = [&](auto pair) __attribute__((always_inline)) {
        constexpr int PI = decltype(pair)::value;
        static_for<2>([&](auto hq) __attribute__((always_inline)) {
          constexpr int h = decltype(hq)::value, t = 2 * PI + h;
          constexpr int s = QT * Q + t, ci = t / KHW, pos = t % KHW;
          float x = qb[B][pos][ci];
          asm volatile("" : "+v"(x));
#pragma unroll
          for (int r = 0; r < R; ++r)
            pr[PI % 2][h][r] = __builtin_amdgcn_mfma_f32_4x4x1f32(wv[S][r][s / 16], x,
                                                                  f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 4, s % 16, 0);
        });
      };
      issue(std::integral_constant<int, 0>{});
      static_for<NP>([&](auto pn) __attribute__((always_inline)) {
        constexpr int n = decltype(pn)::value;
        if constexpr (n + 1 < NP) issue(std::integral_constant<int, n + 1>{});
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] = acc[r] + pr[n % 2][h][r];
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" : "+v"(acc[r]));
      });
    }
  };

  // The loads go out in the order weights c, halo c, weights c+1, halo c+1,
  // ...; each group is fenced so the compiler keeps that order.
  auto fence = []() __attribute__((always_inline)) { asm volatile("" ::: "memory"); };
  // The block's barrier: the wave's own LDS stores done, then s_barrier.
  // (__syncthreads would also wait for the weight loads into LDS, which only
  // the wave that issued them reads, and drain their ring at every chunk.)
  auto barrier = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // prologue: chunk 0 in buffer 0 and its weights in registers, chunk 1's
  // halo (and with three stages its weights) in flight, chunk 0's first
  // quad read
  load_w(0);
  fence();
  load_halo(0, std::integral_constant<int, 0>{});
  fence();
  if constexpr (NWS == 3) {
    load_w(1);
    fence();
  }
  load_halo(1, std::integral_constant<int, 1>{});
  fence();
  barrier();  // the +0 fill before any stage is written
  store_halo(std::integral_constant<int, 0>{}, 0);
  read_w(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 2 * NL + (NWS - 2) * NIW>{});
  barrier();
  read(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, tp);

  ring_loop<2>(0, nch, [&](int c, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;  // c % 2
    fence();
    load_w(c + NWS - 1);
    fence();
    // quad Q of a chunk is in qb[Q % 2] (a chunk has an even number of quads)
    static_for<NQC / 2>([&](auto quad) __attribute__((always_inline)) {
      constexpr int Q = decltype(quad)::value;
      read(std::integral_constant<int, Q + 1>{}, std::integral_constant<int, (Q + 1) % 2>{}, tp);
      __builtin_amdgcn_sched_barrier(0);
      products(quad, par, std::integral_constant<int, Q % 2>{});
    });
    const int nb = (c + 1) % NBUF;
    const int delta = (nb - c % NBUF) * (bufsz / 4);
    if constexpr (NBUF == 3) {
      // chunk c+1 into buffer (c+1) % 3 (last read in chunk c-2, which every
      // wave finished before the barrier of chunk c-1), chunk c+2's loads,
      // the barrier
      store_halo(std::integral_constant<int, 1 - P>{}, nb);
      fence();
      load_halo(c + 2, par);
      fence();
      barrier();
    } else {
      // two buffers: buffer (c+1) % 2 was read in chunk c-1, which every wave
      // has finished at this barrier; a second barrier before the last quad
      // makes chunk c+1's halo visible to its first quad's reads
      barrier();
      store_halo(std::integral_constant<int, 1 - P>{}, nb);
      fence();
      load_halo(c + 2, par);
      fence();
    }
#pragma unroll
    for (int t = 0; t < KH; ++t) tn[t] = tp[t] + delta;
    static_for<NQC - NQC / 2>([&](auto qq) __attribute__((always_inline)) {
      constexpr int Q = NQC / 2 + decltype(qq)::value;
      if constexpr (Q + 1 < NQC) {
        read(std::integral_constant<int, Q + 1>{}, std::integral_constant<int, (Q + 1) % 2>{}, tp);
      } else {
        if constexpr (NBUF == 2) barrier();
        read(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, tn);
        // chunk c+1's weights, before the last quad: after them went halo c+2
        // (three stages: halo c+1, weights c+2 and halo c+2)
        read_w(c + 1, std::integral_constant<int, 1 - P>{},
               std::integral_constant<int, NWS == 2 ? NL : 2 * NL + NIW>{});
      }
      __builtin_amdgcn_sched_barrier(0);
      products(std::integral_constant<int, Q>{}, par, std::integral_constant<int, Q % 2>{});
    });
#pragma unroll
    for (int t = 0; t < KH; ++t) tp[t] = tn[t];
  });

  if (valid) {
    float *base = out_ptr<kBGather>(p, tc.g, 0, img * p.OHW + pix);
    // one uniform test picks the store loop with or without the epilogue
    auto store_all = [&](auto epi) __attribute__((always_inline)) {
      constexpr bool E = decltype(epi)::value;
      float pb[R][RA], pr[R][RA];
      if constexpr (E) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < RA; ++i) {
            const int row = wrow0 + RA * r + i;
            const bool ok = row < p.M;
            pb[r][i] = epi_bias(p, ok, tc.g * p.M + row);
            pr[r][i] = epi_res(p, ok, base + (int64_t)(ok ? row : 0) * p.OHW);
          }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < RA; ++i) {
          const int row = wrow0 + RA * r + i;
          const float v = DPP ? accd[r] : acc[r][i];
          if (row < p.M) {
            if constexpr (E)
              base[(int64_t)row * p.OHW] = finish_with(p, v, pb[r][i], pr[r][i]);
            else
              base[(int64_t)row * p.OHW] = finish<false>(p, v, 0, base);
          }
        }
    };
    if (p.bias == nullptr && p.res == nullptr && p.act == 0)
      store_all(std::false_type{});
    else
      store_all(std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// Panel kernel: fast-mode products whose B rows are read 64 columns at a
// time -- matrix products (KIND kBMatrix), 1x1 convolutions read in place
// (kBPlanes) or through a stride and padding (kBGather) -- on the matrix
// cores, for shapes whose outputs split into enough chains of 4 rows to
// fill the chip.  The chains are the halo kernel's: CW waves over 64
// columns (a convolution's: 64 consecutive output pixels of one image),
// wave w with R chains of 4 rows, one v_mfma_f32_4x4x1_16b_f32 per k step
// and chain, the weights through the A broadcast from the wave's own ring
// of LDS stages.
//
// B is staged in chunks of CC rows (k steps) x 64 columns, straight
// from memory into LDS by the load itself ([row][column]): with BV, 16
// bytes per lane (four columns; a load covers four rows), else 4 bytes (a
// load covers one row, each lane its own column, its own input pixel
// through the stride and padding, or an offset past the buffer for a
// padding tap or a column past the end: +0).  Rows past k are +0 and
// their weights -0 (fast mode's padding).  A chunk's loads are shared by
// the waves, a quarter each, so it is in LDS once every wave's own loads
// are (each waits for its loads by count) and the block has met at a
// barrier.  That barrier sits before the last 16 steps of each chunk's
// products: at it every wave has finished the chunk before, whose stage is
// then reloaded with the chunk NS-1 ahead, so the loads have NS-2 chunks of
// products to arrive in.  (A barrier stops a wave's matrix cores for some
// 200 cycles, hidden only by another block's waves on the same compute
// unit: chunks of 64 steps keep it to about a sixth of the time where one
// block holds a compute unit; chunks of 32 need less LDS, so that two
// blocks share one.)
// ---------------------------------------------------------------------------
template <int KIND, int R, int CW, int CC, int NS, bool BV, bool AV>
__global__ void __launch_bounds__(64 * CW) panel_kernel(Problem p) {
  // CC: k steps per chunk; NS: stages (B and weights)
  constexpr int NG = CC / 16;             // 16-step groups per chunk
  constexpr int BST = CC * 64;            // floats of a B stage
  constexpr int NBL = BV ? CC / 4 / CW : CC / CW;  // B loads per wave and chunk
  constexpr int WROWS = 4 * R, WST = WROWS * CC;    // a wave's weight rows; floats of its stage
  constexpr int WW = AV ? 4 : 1;                    // weight taps per lane and load
  constexpr int NQ = WST / WW, NIW = (NQ + 63) / 64;  // weight loads per wave and chunk
  constexpr int L = NBL + NIW;                      // loads per wave and chunk
  constexpr int LATER = (NS - 3) * L;               // loads issued after a chunk's, at its wait
  static_assert(CC % 16 == 0 && NS >= 3, "panel chunk shape");
  static_assert(NBL >= 1 && (BV ? (CC / 4) % CW == 0 : CC % CW == 0), "panel chunk shape");
  static_assert((NS - 2) * L <= 63, "load count");
  // [NS][CC][64] B, then per wave [NS][WROWS][CC] weights
  extern __shared__ __align__(16) float ss[];

  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr bool CONV = KIND != kBMatrix;
  // the tile's columns
  int img = 0, col0;
  if constexpr (CONV) {
    const int tpi = (p.OHW + 63) / 64;
    img = tc.tn / tpi;
    col0 = (tc.tn - img * tpi) * 64;
  } else {
    col0 = tc.tn * 64;
  }
  const int ncols = CONV ? p.OHW : p.N;
  const bool valid = col0 + lane < ncols;
  // B: rows of the chunk at bbase + row * rstride (floats)
  const float *bbase = CONV ? p.B + img * p.x_img + tc.g * p.x_grp : p.B;
  const int64_t rstride = CONV ? (int64_t)p.HW : p.ldb;
  uint32_t boff[BV ? NBL : 1];  // BV: byte offset of each load's quad within the chunk (or kOutside)
  int brow[BV ? NBL : 1];       // BV: its row within the chunk
  uint32_t coff = kOutside;     // 4-byte loads: the lane's column within a row
  const uint32_t rstep = (uint32_t)(rstride * 4);  // bytes between rows
  if constexpr (BV) {
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      const int qd = (wave * NBL + j) * 64 + lane;  // quad of the chunk: row qd / 16, columns 4 (qd % 16)
      brow[j] = qd / 16;
      const int c = col0 + 4 * (qd % 16);
      boff[j] = c < ncols ? (uint32_t)(((int64_t)brow[j] * rstride + c) * 4) : kOutside;
    }
  } else if constexpr (KIND == kBGather) {
    const int oy = valid ? (col0 + lane) / p.OW : 0;
    const int ox = valid ? col0 + lane - oy * p.OW : 0;
    const int iy = oy * p.sH - p.pT, ix = ox * p.sW - p.pL;
    if (valid && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W)
      coff = (uint32_t)(4 * (iy * p.W + ix));
  } else {
    if (valid) coff = (uint32_t)(4 * (col0 + lane));
  }
  const bool col_in = coff != kOutside;

  // the wave's weight rows, as in the halo kernel
  const int wrow0 = tc.tm * (4 * R * CW) + wave * 4 * R;
  const int wbase = min(wrow0, p.M - 1);
  const __amdgpu_buffer_rsrc_t wrs =
      buffer_at(p.A + tc.g * p.a_gstride + (int64_t)wbase * p.lda, kRange);
  float *const wring = ss + NS * BST + wave * NS * WST;
  uint32_t wq[NIW];
  int wt[NIW];
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int q = n * 64 + lane, r = q / (CC / WW);
    wt[n] = (q - r * (CC / WW)) * WW;
    wq[n] = q < NQ && wrow0 + r < p.M
                ? (uint32_t)((int64_t)(wrow0 + r - wbase) * p.lda * 4 + 4 * wt[n])
                : kOutside;
  }
  const int tb = lane >> 2;  // the lane's tap within a 16-step group
  const int nch = (p.K + CC - 1) / CC, last = nch - 1;
  typedef __attribute__((address_space(3))) void lds_t;

  // chunk c's B (this wave's share) and weights into stage c % NS
  auto load = [&](int c) __attribute__((always_inline)) {
    const int k0 = min(c, last) * CC, st = c % NS;
    if constexpr (BV) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(bbase + (int64_t)k0 * rstride, kRange);
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        const uint32_t off = k0 + brow[j] < p.K ? boff[j] : kOutside;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t *)(ss + st * BST + (wave * NBL + j) * 256),
                                                 16, off, 0, 0, 0);
      }
    } else {
      // the wave's rows from row0 of the chunk: the lane's offset advances by
      // one row per load (carried in one register; used only where the
      // lane's column is inside, so it never wraps into range)
      const int row0 = wave * NBL, rows_left = p.K - k0 - row0;  // uniform
      const __amdgpu_buffer_rsrc_t rs = buffer_at(bbase + ((int64_t)k0 + row0) * rstride, kRange);
      uint32_t vo = coff;
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t *)(ss + st * BST + (row0 + j) * 64), 4,
                                                 col_in && j < rows_left ? vo : kOutside, 0, 0, 0);
        vo += rstep;
      }
    }
    float *dst = wring + st * WST;
#pragma unroll
    for (int n = 0; n < NIW; ++n) {
      const uint32_t off = wq[n] != kOutside && k0 + wt[n] < p.K ? wq[n] + 4 * k0 : kOutside;
      if (NQ % 64 == 0 || n + 1 < NIW || lane < NQ % 64) {
        auto *to = (lds_t *)(dst + n * 64 * WW);
        if constexpr (AV)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, to, 16, off, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, to, 4, off, 0, 0, 0);
      }
    }
  };
  auto fence = []() __attribute__((always_inline)) { asm volatile("" ::: "memory"); };
  auto wait_and_meet = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(LATER) : "memory");
  };

  float wv[2][R][NG];  // weights of chunk c in slot c % 2
  float bv[2][16];     // B values of a group, read one group ahead
  f32x4 acc[R];
#pragma unroll
  for (int c = 0; c < R; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // chunk c's weights into slot S; in a chunk running past k (the last one
  // at most) the wave first writes -0 over its stage's steps past k (its own
  // stage: its LDS operations run in order, no wait)
  auto read_w = [&](int c, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    float *stg = wring + (c % NS) * WST;
    if ((c + 1) * CC > p.K) {
      for (int e = lane; e < WST; e += 64)
        if (c * CC + e % CC >= p.K) stg[e] = -0.0f;
    }
    const float *src = stg + (lane & 3) * CC + tb;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int g = 0; g < NG; ++g) wv[S][r][g] = src[4 * r * CC + 16 * g];
  };
  auto read = [&](int c, auto grp, auto into) __attribute__((always_inline)) {
    constexpr int G = decltype(grp)::value, B = decltype(into)::value;
    const float *src = ss + (c % NS) * BST + lane;
    static_for<16>([&](auto uq) __attribute__((always_inline)) {
      constexpr int u = decltype(uq)::value;
      bv[B][u] = src[(16 * G + u) * 64];
    });
  };
  auto products = [&](auto grp, auto slot, auto from) __attribute__((always_inline)) {
    constexpr int G = decltype(grp)::value, S = decltype(slot)::value, B = decltype(from)::value;
    static_for<16>([&](auto uq) __attribute__((always_inline)) {
      constexpr int u = decltype(uq)::value;
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_4x4x1f32(wv[S][r][G], bv[B][u], acc[r], 4, u, 0);
    });
  };

  // k = 0: no chunk, nothing to load (chunk indices below would be negative)
  if (nch > 0) {
  // prologue: chunks 0 .. NS-2 in flight, then chunk 0 in
#pragma unroll
  for (int c = 0; c < NS - 1; ++c) {
    fence();
    load(c);
  }
  fence();
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"((NS - 2) * L) : "memory");
  read_w(0, std::integral_constant<int, 0>{});
  read(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});

  // group G of chunk c is read into bv[(P*NG + G) % 2], P = c % 2
  ring_loop<2>(0, nch, [&](int c, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    static_for<NG - 1>([&](auto grp) __attribute__((always_inline)) {
      constexpr int G = decltype(grp)::value;
      read(c, std::integral_constant<int, G + 1>{}, std::integral_constant<int, (P * NG + G + 1) % 2>{});
      __builtin_amdgcn_sched_barrier(0);
      products(grp, par, std::integral_constant<int, (P * NG + G) % 2>{});
    });
    // chunk c+1: this wave's loads of it in (after them went chunks
    // c+2 .. c+NS-2), then the block's barrier; chunk c-1's stage is free
    fence();
    wait_and_meet();
    load(c + NS - 1);
    fence();
    read_w(c + 1, std::integral_constant<int, 1 - P>{});
    constexpr int G = NG - 1;
    read(c + 1, std::integral_constant<int, 0>{}, std::integral_constant<int, (P * NG + G + 1) % 2>{});
    __builtin_amdgcn_sched_barrier(0);
    products(std::integral_constant<int, G>{}, par, std::integral_constant<int, (P * NG + G) % 2>{});
  });
  }

  if (valid) {
    float *base = out_ptr<KIND>(p, tc.g, 0, CONV ? img * p.OHW + col0 + lane : col0 + lane);
    const int64_t rs = CONV ? (int64_t)p.OHW : p.ldc;
    auto store_all = [&](auto epi) __attribute__((always_inline)) {
      constexpr bool E = decltype(epi)::value;
      float pb[R][4], pr[R][4];
      if constexpr (E) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = wrow0 + 4 * r + i;
            const bool ok = row < p.M;
            pb[r][i] = epi_bias(p, ok, tc.g * p.M + row);
            pr[r][i] = epi_res(p, ok, base + (int64_t)(ok ? row : 0) * rs);
          }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wrow0 + 4 * r + i;
          if (row < p.M) {
            if constexpr (E)
              base[(int64_t)row * rs] = finish_with(p, acc[r][i], pb[r][i], pr[r][i]);
            else
              base[(int64_t)row * rs] = finish<false>(p, acc[r][i], 0, base);
          }
        }
    };
    if (p.bias == nullptr && p.res == nullptr && p.act == 0)
      store_all(std::false_type{});
    else
      store_all(std::true_type{});
  }
}

// ---------------------------------------------------------------------------
// Depthwise kernel: Cin/G = 1, any channel multiplier Cout/G.  The pages run
// depthwise convolutions on a kernel of their own that computes the
// convolution expression directly ("Matrix product and convolution
// kernels", section "Convolution"; "Exact mode", section "Convolution"):
// output (n, oc, oy, ox) of group g = oc / (Cout/G) is the sum over (ky, kx),
// kernel row then kernel column, of w[oc][0][ky][kx] * x[n][g][iy][ix], +0
// outside the plane.  With only KH*KW terms per output the work is bound by
// moving x and y, not by arithmetic, so there are no matrix cores and no LDS
// tiles here: a wave owns 64 consecutive output pixels of one (image, output
// channel) plane, its channel's weights are wave-uniform (read once into
// registers), and each lane runs its own output's terms in order, a tap being
// one buffer load of the input plane at a byte offset that lies past the
// plane's range for a padding tap (read as +0, never stored).  Neighbouring
// lanes read neighbouring input pixels, so the taps of a window come from the
// same cache lines.  KH_ = KW_ = 0: the window size is read at run time.
// A lane computes P outputs 64 pixels apart (P = 2 or 4 on larger planes), so
// one round of resident waves covers a layer and each wave has P*KH*KW loads
// in flight.  Launch: tiles_m = waves per output plane (64*P pixels each),
// tiles_n = N*Cout planes, four waves per block, blocks numbered so that each
// XCD runs a contiguous range of waves (the waves of a plane share its input
// rows in one L2).
// ---------------------------------------------------------------------------
__device__ inline int xcd_contiguous(int bid, int nblocks) {
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

template <int MODE>
__device__ __forceinline__ float term(float acc, float w, float v) {
  if (MODE == kFast) return __builtin_fmaf(w, v, acc);
  const float prod = w * v;
  return acc + prod;
}

template <int MODE, int KH_, int KW_, int P, bool EPI>
__global__ void __launch_bounds__(256) dw_kernel(Problem p) {
  static_assert(P == 1 || (KH_ > 0 && KW_ > 0), "several outputs per lane: compiled windows only");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(xcd_contiguous(blockIdx.x, gridDim.x) * 4 + (tid >> 6));
  const int plane = wv / p.tiles_m;  // image * Cout + output channel
  if (plane >= p.tiles_n) return;    // whole waves past the last plane
  const int cout = p.groups * p.M;
  const int img = plane / cout, oc = plane - img * cout, g = oc / p.M;
  const __amdgpu_buffer_rsrc_t rs =
      buffer_at(p.B + img * p.x_img + (int64_t)g * p.HW, 4u * (uint32_t)p.HW);
  const float *wp = p.A + (int64_t)oc * p.KHW;  // row oc of the weights, KH*KW taps
  // output j of this lane: pixel pix0 + 64 j of the plane
  const int pix0 = (wv - plane * p.tiles_m) * (64 * P) + lane;
  int iy0[P], ix0[P];
  bool valid[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int pix = pix0 + 64 * j;
    valid[j] = pix < p.OHW;
    const int oy = valid[j] ? pix / p.OW : 0, ox = valid[j] ? pix - oy * p.OW : 0;
    iy0[j] = oy * p.sH - p.pT;
    ix0[j] = ox * p.sW - p.pL;
  }
  // byte offset of tap (ky, kx) of output j in the plane, or past its range
  auto offset = [&](int j, int ky, int kx) __attribute__((always_inline)) {
    const int iy = iy0[j] + ky * p.dH, ix = ix0[j] + kx * p.dW;
    const bool in = valid[j] & ((unsigned)iy < (unsigned)p.H) & ((unsigned)ix < (unsigned)p.W);
    // unsigned: for a tap outside the plane the product may wrap, and is not used
    const uint32_t o = 4u * ((uint32_t)iy * (uint32_t)p.W + (uint32_t)ix);
    return in ? o : kOutside;
  };
  float acc[P];
#pragma unroll
  for (int j = 0; j < P; ++j) acc[j] = 0.0f;
  if constexpr (KH_ > 0) {
    constexpr int T = KH_ * KW_;
    float w[T], v[P][T];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int ky = 0; ky < KH_; ++ky)
#pragma unroll
        for (int kx = 0; kx < KW_; ++kx) v[j][ky * KW_ + kx] = load1(rs, offset(j, ky, kx));
#pragma unroll
    for (int t = 0; t < T; ++t) w[t] = wp[t];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[j] = term<MODE>(acc[j], w[t], v[j][t]);
  } else {
    for (int ky = 0; ky < p.KH; ++ky)
      for (int kx = 0; kx < p.KW; ++kx)
        acc[0] = term<MODE>(acc[0], wp[ky * p.KW + kx], load1(rs, offset(0, ky, kx)));
  }
  float *yp = p.C + img * p.y_img + (int64_t)oc * p.OHW;
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (valid[j]) yp[pix0 + 64 * j] = finish<EPI>(p, acc[j], oc, yp + pix0 + 64 * j);
}

// ---------------------------------------------------------------------------
// Depthwise kernel, band form (planes at least 28 pixels wide, 3x3 or 5x5
// windows).  A block of 256 threads owns BH output rows of one (image,
// output channel) plane.  It first stages the input rows those outputs read
// (IH = (BH-1)*sH + (KH-1)*dH + 1 rows of IW = (OW-1)*sW + (KW-1)*dW + 1
// columns, starting at the band's first window origin) in LDS, each element
// one load of a contiguous row segment, +0 for the padding (written into
// LDS, never stored in memory); then each thread runs the chains of its
// outputs, taps read from LDS in (ky, kx) order.  Every input element is
// loaded once per band instead of once per tap, which is what the strided
// and 5x5 windows are bound by in the one-wave-per-64-pixels form.
// Launch: tiles_m = bands per plane, tiles_n = N*Cout planes, dynamic LDS
// 4*IH*IW bytes.
// ---------------------------------------------------------------------------
template <int MODE, int KH, int KW, bool EPI>
__global__ void __launch_bounds__(256) dw_band_kernel(Problem p) {
  extern __shared__ float tile[];
  const int tid = threadIdx.x;
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x);
  const int plane = blk / p.tiles_m, band = blk - plane * p.tiles_m;
  const int cout = p.groups * p.M;
  const int img = plane / cout, oc = plane - img * cout, g = oc / p.M;
  const int oy0 = band * p.bh;
  const int iy0 = oy0 * p.sH - p.pT, ix0 = -p.pL;
  const __amdgpu_buffer_rsrc_t rs =
      buffer_at(p.B + img * p.x_img + (int64_t)g * p.HW, 4u * (uint32_t)p.HW);
  // stage the band, 8 elements per thread per batch (all loads of a batch in
  // flight); element e = (r, c) of the tile, stepped by 256 without division
  const int total = p.ih * p.iw;
  const int dr = 256 / p.iw, dc = 256 - dr * p.iw;
  int r = tid / p.iw, c = tid - r * p.iw;
  for (int e0 = 0; e0 < total; e0 += 8 * 256) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int iy = iy0 + r, ix = ix0 + c;
      const bool in = (e0 + i * 256 + tid < total) & ((unsigned)iy < (unsigned)p.H) &
                      ((unsigned)ix < (unsigned)p.W);
      v[i] = load1(rs, in ? 4u * ((uint32_t)iy * (uint32_t)p.W + (uint32_t)ix) : kOutside);
      r += dr;
      c += dc;
      if (c >= p.iw) {
        c -= p.iw;
        ++r;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * 256 + tid;
      if (e < total) tile[e] = v[i];
    }
  }
  __syncthreads();
  const float *wp = p.A + (int64_t)oc * p.KHW;
  float w[KH * KW];
#pragma unroll
  for (int t = 0; t < KH * KW; ++t) w[t] = wp[t];
  const int rows = min(p.bh, p.OHW / p.OW - oy0);
  const int nout = rows * p.OW;
  float *yp = p.C + img * p.y_img + (int64_t)oc * p.OHW + (int64_t)oy0 * p.OW;
  // output o = (oyl, ox) of the band, stepped by 256 without division
  const int qr = 256 / p.OW, qc = 256 - qr * p.OW;
  int oyl = tid / p.OW, ox = tid - oyl * p.OW;
  for (int o = tid; o < nout; o += 256) {
    const float *t = tile + oyl * p.sH * p.iw + ox * p.sW;
    float acc = 0.0f;
#pragma unroll
    for (int ky = 0; ky < KH; ++ky)
#pragma unroll
      for (int kx = 0; kx < KW; ++kx)
        acc = term<MODE>(acc, w[ky * KW + kx], t[ky * p.dH * p.iw + kx * p.dW]);
    yp[o] = finish<EPI>(p, acc, oc, yp + o);
    oyl += qr;
    ox += qc;
    if (ox >= p.OW) {
      ox -= p.OW;
      ++oyl;
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped direct kernel: a grouped 3x3 convolution with few output channels
// per group (Cout/G <= 8; the grouped, dilated workload; ResNeXt-style
// blocks).  Each output is the convolution expression of "Exact mode",
// section "Convolution": its terms in (c, ky, kx) order from +0.  The
// implicit product would give such a group an 8-row tile; here a wave owns 64
// consecutive output pixels of one (image, group) and each lane keeps all R
// (>= Cout/G) output channels of its pixel, so a tap, loaded once (a buffer
// load at the pixel's offset in channel c's plane, or past the plane for a
// padding tap, +0), feeds R terms.  Channels are loaded 8 at a time (72 tap
// loads in flight per lane); their taps, in (c, ky, kx) order, run in chunks
// of 16 through dpp_steps, two rows at a time, the weights of a row's chunk
// in one register (lane u of each row of 16 holds tap k0 + u) broadcast by
// DPP.  Taps past the group (the padding of the last chunk) read +0 on both
// sides, so their terms leave the sums unchanged; rows past Cout/G read +0
// weights and are not stored.
// Launch: tiles_m = waves per (image, group), tiles_n = N*G, 4 waves per block.
// ---------------------------------------------------------------------------
template <int MODE, int KH, int KW, int R, bool EPI>
__global__ void __launch_bounds__(256) grouped_kernel(Problem p) {
  constexpr int T = KH * KW, CB = 8, NT = CB * T, NQ = (NT + 15) / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(xcd_contiguous(blockIdx.x, gridDim.x) * 4 + (tid >> 6));
  const int item = wv / p.tiles_m;  // image * G + group
  if (item >= p.tiles_n) return;    // whole waves past the last (image, group)
  const int img = item / p.groups, g = item - img * p.groups;
  const int pix = (wv - item * p.tiles_m) * 64 + lane;
  const bool valid = pix < p.OHW;
  const int oy = valid ? pix / p.OW : 0, ox = valid ? pix - oy * p.OW : 0;
  const int iy0 = oy * p.sH - p.pT, ix0 = ox * p.sW - p.pL;
  uint32_t voff[T];
#pragma unroll
  for (int ky = 0; ky < KH; ++ky)
#pragma unroll
    for (int kx = 0; kx < KW; ++kx) {
      const int iy = iy0 + ky * p.dH, ix = ix0 + kx * p.dW;
      const bool in = valid & ((unsigned)iy < (unsigned)p.H) & ((unsigned)ix < (unsigned)p.W);
      voff[ky * KW + kx] = in ? 4u * ((uint32_t)iy * (uint32_t)p.W + (uint32_t)ix) : kOutside;
    }
  const float *xg = p.B + img * p.x_img + g * p.x_grp;  // channel 0 of the group
  const __amdgpu_buffer_rsrc_t rw = buffer_at(p.A + g * p.a_gstride, kRange);  // the group's weights
  const int cin_g = p.K / T;
  constexpr int RP = R >= 2 ? R / 2 : 1;  // row pairs (R = 1: one row)
  float acc[RP][R >= 2 ? 2 : 1];
#pragma unroll
  for (int i = 0; i < RP; ++i)
#pragma unroll
    for (int j = 0; j < (R >= 2 ? 2 : 1); ++j) acc[i][j] = 0.0f;
  for (int c0 = 0; c0 < cin_g; c0 += CB) {
    float v[NQ * 16];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = c0 + j;  // a channel past the group reads +0 (empty range)
      const __amdgpu_buffer_rsrc_t rs =
          buffer_at(xg + (int64_t)min(c, cin_g - 1) * p.HW, c < cin_g ? 4u * (uint32_t)p.HW : 0u);
#pragma unroll
      for (int t = 0; t < T; ++t) v[j * T + t] = load1(rs, voff[t]);
    }
#pragma unroll
    for (int k = NT; k < NQ * 16; ++k) v[k] = 0.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int k = c0 * T + q * 16 + (lane & 15);  // this lane's weight tap in the chunk
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        constexpr int RR = R >= 2 ? 2 : 1;
        float w[RR];
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          const int row = i * RR + j;
          const bool tap = k < p.K && q * 16 + (lane & 15) < NT;
          const bool ok = row < p.M && tap;
          w[j] = load1(rw, ok ? (uint32_t)(4 * ((int64_t)row * p.lda + k)) : kOutside);
          // fast mode, a tap past the group (its input reads +0): weight
          // -0, so the term adds a product of -0, which leaves any sum
          // unchanged
          if (MODE == kFast) w[j] = or_sign(w[j], pad_sign(!tap));
        }
        dpp_steps<MODE, RR, 16>(acc[i], w, &v[q * 16]);
      }
    }
  }
  if (valid) {
    float *yp = p.C + img * p.y_img + (int64_t)g * p.y_grp + pix;
#pragma unroll
    for (int i = 0; i < RP; ++i)
#pragma unroll
      for (int j = 0; j < (R >= 2 ? 2 : 1); ++j) {
        const int row = i * (R >= 2 ? 2 : 1) + j;
        if (row < p.M)
          yp[(int64_t)row * p.OHW] = finish<EPI>(p, acc[i][j], g * p.M + row, yp + (int64_t)row * p.OHW);
      }
  }
}

// ---------------------------------------------------------------------------
// Row-dot kernel: out_g[r] = sum over p of W_g[r][p] * v_g[p], p increasing,
// for rows W whose k taps are contiguous.  It serves the single-column
// products: one row times the transpose of an N x K matrix (m = 1), and,
// with short rows, a matrix times one column (n = 1) and the 1x1
// convolutions of a 1x1 input at batch 1, the squeeze-and-excitation layers
// ("Convolution (fast mode)", section "Single-column products").  Every
// output is still one lane's chain over the whole of k from +0 ("Exact
// mode", matrix product).  A lane owns one row and streams it in chunks of
// 16 taps through a ring of D chunks of registers (16-byte loads when rows
// are 16-byte aligned); lane u of each row of 16 lanes holds tap k0 + u of
// v, which the DPP broadcast of dpp_steps hands to every lane, so a chunk is
// 16 dependent steps with no LDS and no barrier.  Taps past k read +0 on both
// sides.  One wave per block (64 rows), blocks spread over the XCDs.  Each
// load instruction reads 16 bytes of 64 different rows, which holds a long
// row's stream to the texture units' rate of distinct lines.
//   W_g row r at A + g*a_gstride + r*lda;  v_g tap t at B + g*x_grp + t*ldb;
//   out_g[r] at C + g*y_grp + r*ldc.
// ---------------------------------------------------------------------------
template <int MODE, bool VEC, int D>
__global__ void __launch_bounds__(64) rowdot_kernel(Problem p) {
  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, 1);
  const int lane = threadIdx.x;
  const int row0 = tc.tm * 64;  // the wave's first row
  const bool ok = row0 + lane < p.M;
  const float *wbase = p.A + tc.g * p.a_gstride + (int64_t)row0 * p.lda;
  const float *vbase = p.B + tc.g * p.x_grp;
  const uint32_t roff = ok ? (uint32_t)(4 * (int64_t)lane * p.lda) : kOutside;
  const uint32_t voff = (uint32_t)(4 * (int64_t)(lane & 15) * p.ldb);
  const int nchunks = (p.K + 15) / 16, last = nchunks - 1;
  float wr[D][16], vr[D];
  float acc[1] = {0.0f};
  auto load = [&](int c, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int k0 = c * 16;
    const __amdgpu_buffer_rsrc_t rw = buffer_at(wbase + k0, kRange);
    if constexpr (VEC) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        load4(rw, ok && k0 + 4 * q < p.K ? roff + 16 * q : kOutside, &wr[S][4 * q]);
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) wr[S][t] = load1(rw, ok && k0 + t < p.K ? roff + 4 * t : kOutside);
    }
    const __amdgpu_buffer_rsrc_t rv = buffer_at(vbase + (int64_t)k0 * p.ldb, kRange);
    vr[S] = load1(rv, k0 + (lane & 15) < p.K ? voff : kOutside);
  };
  // chunk c; in fast mode the row's taps at or beyond K are -0 (v's are +0),
  // so each padded term adds a product of -0.  Only the chunk that runs past
  // K has such taps (a uniform test): the sign fix costs the other chunks'
  // chains nothing.
  auto compute = [&](auto slot, int c) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const float w1[1] = {vr[S]};
    if constexpr (MODE == kFast) {
      if ((c + 1) * 16 > p.K) {
#pragma unroll
        for (int t = 0; t < 16; ++t) wr[S][t] = or_sign(wr[S][t], pad_sign(c * 16 + t >= p.K));
      }
    }
    dpp_steps<MODE, 1, 16>(acc, w1, wr[S]);
  };
  if (nchunks > 0) {
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) { load(min((int)decltype(j)::value, last), j); });
    const int full = nchunks - nchunks % D;
    for (int c0 = 0; c0 < full; c0 += D) {
      static_for<D>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        load(min(c0 + J + D - 1, last), std::integral_constant<int, (J + D - 1) % D>{});
        compute(j, c0 + J);
      });
    }
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) {
      if (full + (int)decltype(j)::value < nchunks) compute(j, full + (int)decltype(j)::value);
    });
  }
  if (ok) {
    float *d = p.C + tc.g * p.y_grp + (int64_t)(row0 + lane) * p.ldc;
    *d = finish(p, acc[0], tc.g * p.M + row0 + lane, d);
  }
}


// The end of a split-k block: the KS partial tiles meet in LDS (element (row,
// col) of wave w at red[w * BM * BN + row * BN + col]); each thread adds its
// outputs' partial sums in wave order and stores them through the epilogue.
template <int KIND, int TM, int TN, int KS>
__device__ __forceinline__ void splitk_finish(const Problem &p, int g, int m0, int n0, int wave,
                                              const f32x4 (&acc)[TM][TN], float *red) {
  constexpr int BM = 16 * TM, BN = 16 * TN;
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[wave * BM * BN + (16 * i + 4 * lg + r) * BN + 16 * j + li] = acc[i][j][r];
  __syncthreads();
  const bool epi = p.bias != nullptr || p.res != nullptr || p.act != 0;
  for (int o = threadIdx.x; o < BM * BN; o += 64 * KS) {
    const int row = o / BN, col = o - (o / BN) * BN;
    const int gr = m0 + row, gc = n0 + col;
    if (gr >= p.M || gc >= p.N) continue;
    float v = red[o];
#pragma unroll
    for (int w = 1; w < KS; ++w) v += red[w * BM * BN + o];
    float *d = out_ptr<KIND == kBMatrixT ? kBMatrix : KIND>(p, g, gr, gc);
    *d = epi ? finish(p, v, g * p.M + gr, d) : canonical(v);
  }
}

// ---------------------------------------------------------------------------
// Split-k matrix-core kernel: fast mode under a stated tolerance (mode 2).
// Every output is still one sum over all of k, but the order of its terms is
// not fixed: v_mfma_f32_16x16x4_f32 adds four products at once (its internal
// order and roundings are not specified), and the KS waves of a block each
// sum a contiguous range of k, their partial sums then added in wave order.
// What is promised instead of bits is the bound |c - r| <= 4e-6 * sqrt(K) *
// sum |a*b| + 1e-30 against the exact sum r (the sequential-summation bound
// k*u*sum|a*b| of "Matrix product and convolution kernels", section "Fast
// mode", in the 4e-6*sqrt(K) form of the dotLLM pull request "F32
// outer-product tiled GEMM kernel for prefill", section "Tests"), and the
// class of a non-finite exact result.  Results repeat from run to run: no
// atomics, and the partial sums are added in a fixed order.
//
// A block of KS waves owns a (16 TM) x (16 TN) output tile of one group;
// wave w sums the chunks of 16 taps [w*per, (w+1)*per).  Operands go from
// memory straight into registers in the instruction's layout, with no LDS
// staging and no barrier until the end: lane l brings A row l % 16 and B
// column l % 16 of each 16 x 16 block for taps 4*(l/16) .. 4*(l/16) + 3 of
// the chunk (one 16-byte load of an aligned A row), and instruction s of the
// chunk takes tap 4*(l/16) + s: the chunk's 16 taps in a permuted order, the
// same on both sides.  Rows, columns and taps beyond the problem read +0.
// Register r of lane l of a block's accumulator holds row 4*(l/16) + r and
// column l % 16 (measured on gfx950).  The partial tiles meet in LDS, where
// each thread adds its outputs' KS partial sums in wave order and stores
// them through the epilogue.  KH, KW: a gathered convolution's window known
// at compile time (0: read at run time).
// ---------------------------------------------------------------------------
template <int KIND, bool AVEC, bool BVEC, int TM, int TN, int KS, int KH, int KW>
__global__ void __launch_bounds__(64 * KS) splitk_kernel(Problem p) {
  // ring of four chunks: three in flight while one is multiplied
  constexpr int BM = 16 * TM, BN = 16 * TN, D = 4;
  __shared__ float red[KS * BM * BN];
  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nch = (p.K + 15) / 16;
  const int per = (nch + KS - 1) / KS;
  const int cb = min(nch, wave * per), ce = min(nch, cb + per);  // this wave's chunks

  // A: rows m0 + 16 i + li, byte offsets from the chunk's first tap
  const float *abase = p.A + tc.g * p.a_gstride + (int64_t)m0 * p.lda;
  uint32_t aoff[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    aoff[i] = m0 + 16 * i + li < p.M ? (uint32_t)(4 * ((16 * i + li) * p.lda + 4 * lg)) : kOutside;

  // B: columns n0 + 16 j + li
  constexpr bool PLANES = KIND == kBPlanes;
  constexpr bool BT = KIND == kBMatrixT, BM_ = KIND == kBMatrix;
  uint32_t boff[TN];   // matrix: byte offset of (tap 4 lg, column) from the chunk base;
                       // planes: of (tap 0, column) from the group's input; past N: kOutside
  int eimg[TN], iy0[TN], ix0[TN];  // gather: image offset and window origin of the column
  bool bok[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + 16 * j + li;
    bok[j] = col < p.N;
    if constexpr (BM_) {
      boff[j] = bok[j] ? (uint32_t)(4 * ((int64_t)(4 * lg) * p.ldb + 16 * j + li)) : kOutside;
    } else if constexpr (BT) {
      boff[j] = bok[j] ? (uint32_t)(4 * ((int64_t)(16 * j + li) * p.ldb + 4 * lg)) : kOutside;
    } else {
      const int cc = bok[j] ? col : 0;
      const int img = cc / p.OHW, pix = cc - img * p.OHW;
      if constexpr (PLANES) {
        boff[j] = (uint32_t)(4 * (img * p.x_img + pix));
      } else {
        const int oy = pix / p.OW, ox = pix - oy * p.OW;
        eimg[j] = (int)(img * p.x_img);
        iy0[j] = oy * p.sH - p.pT;
        ix0[j] = ox * p.sW - p.pL;
      }
    }
  }
  const float *bgrp = p.B + tc.g * p.x_grp;  // convolution: the group's input channels
  const int khw = KH > 0 ? KH * KW : p.KHW, kw = KH > 0 ? KW : p.KW;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float ra[D][TM][4], rb[D][TN][4];

  auto load = [&](int c, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int k0 = c * 16;
    const int kleft = p.K - k0;  // taps of the chunk that exist (may be <= 0: reload past the end)
    // A: four taps of a row, 16 bytes or one by one
    {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(abase + k0, kRange);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (AVEC) {
          load4(rs, 4 * lg < kleft ? aoff[i] : kOutside, ra[S][i]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ra[S][i][e] = load1(rs, 4 * lg + e < kleft && aoff[i] != kOutside ? aoff[i] + 4 * e : kOutside);
        }
      }
    }
    if constexpr (BM_) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(p.B + (int64_t)k0 * p.ldb + n0, kRange);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rb[S][j][e] = load1(rs, 4 * lg + e < kleft && bok[j] ? boff[j] + (uint32_t)(4 * e * p.ldb) : kOutside);
    } else if constexpr (BT) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(p.B + (int64_t)n0 * p.ldb + k0, kRange);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BVEC) {
          load4(rs, 4 * lg < kleft ? boff[j] : kOutside, rb[S][j]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rb[S][j][e] = load1(rs, 4 * lg + e < kleft && bok[j] ? boff[j] + 4 * e : kOutside);
        }
      }
    } else if constexpr (PLANES) {
      const __amdgpu_buffer_rsrc_t rs = buffer_at(bgrp, kRange);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = k0 + 4 * lg + e;  // the input plane of the tap
          rb[S][j][e] = load1(rs, t < p.K && bok[j] ? boff[j] + (uint32_t)(4 * t * p.HW) : kOutside);
        }
    } else {
      // gather: tap t -> (channel, kernel row, kernel column), then the pixel
      // the tap reads, +0 in the padding
      const __amdgpu_buffer_rsrc_t rs = buffer_at(bgrp, kRange);
      const int t0 = k0 + 4 * lg;
      int ch = t0 / khw;
      const int rr = t0 - ch * khw;
      int ky = rr / kw, kx = rr - (rr / kw) * kw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int iy = iy0[j] + ky * p.dH, ix = ix0[j] + kx * p.dW;
          const bool in = bok[j] && t < p.K && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
          rb[S][j][e] = load1(rs, in ? (uint32_t)(4 * (eimg[j] + ch * p.HW + iy * p.W + ix)) : kOutside);
        }
        if (++kx == kw) {
          kx = 0;
          if (++ky * kw == khw) {
            ky = 0;
            ++ch;
          }
        }
      }
    }
  };
  auto compute = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[S][i][e], rb[S][j][e], acc[i][j], 0, 0, 0);
  };
  // a ring of D chunks in flight; loads past the wave's last chunk reload it
  // (branch-free, so each wait is for the loads of D-1 chunks earlier)
  const int n = ce - cb;
  if (n > 0) {
    const int last = ce - 1;
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) { load(min(cb + (int)decltype(j)::value, last), j); });
    const int full = n - n % D;
    for (int c = 0; c < full; c += D) {
      static_for<D>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        load(min(cb + c + J + D - 1, last), std::integral_constant<int, (J + D - 1) % D>{});
        compute(j);
      });
    }
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) {
      if (full + (int)decltype(j)::value < n) compute(j);
    });
  }

  splitk_finish<KIND, TM, TN, KS>(p, tc.g, m0, n0, wave, acc, red);
}

// ---------------------------------------------------------------------------
// Split-k kernel for a gathered convolution whose window (KH x KW > 1) is
// known at compile time, mode 2.  A chunk is four input channels, one per
// lane group (l / 16), times the KH*KW window positions: instruction e of a
// chunk multiplies window position e of the four channels, so each output
// still receives every term once, in an order mode 2 leaves free.  A lane's
// byte offsets for the window positions of its output pixel, image included
// (or past the range, for a padding tap), are computed once; a chunk moves
// only the uniform base of the input and weight buffers by four channels,
// and a lane whose channel lies past the group's last reads past the range.  A lane's weights for a chunk are the KH*KW
// consecutive taps of its channel (12-byte loads when KH*KW is a multiple
// of 3).
// ---------------------------------------------------------------------------
template <bool AVEC, int TM, int TN, int KS, int KH, int KW>
__global__ void __launch_bounds__(64 * KS) splitk_conv_kernel(Problem p) {
  // ring of three chunks (a chunk is 4 * KHW taps: two in flight keep enough
  // loads outstanding; two for the largest tiles, for registers)
  constexpr int KHW = KH * KW, BM = 16 * TM, BN = 16 * TN, D = TM * TN >= 8 ? 2 : 3;
  static_assert(KHW > 1 && 4 * KHW * 4 <= 256, "windows of more than one tap, offsets past kOutside");
  __shared__ float red[KS * BM * BN];
  const TileCoord tc = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int cin_g = p.K / KHW;
  const int nch = (cin_g + 3) / 4;  // chunks of four channels
  const int per = (nch + KS - 1) / KS;
  const int cb = min(nch, wave * per), ce = min(nch, cb + per);

  // weights: row m0 + 16 i + li, channel 4 c + lg: KHW taps at this offset
  // from the chunk's base (rows past M: past the range)
  const float *abase = p.A + tc.g * p.a_gstride + (int64_t)m0 * p.lda;
  uint32_t aoff[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    aoff[i] = m0 + 16 * i + li < p.M ? (uint32_t)(4 * ((16 * i + li) * p.lda + lg * KHW)) : kOutside;
  // input: column n0 + 16 j + li, window position e: offset of channel lg's
  // pixel in the column's image (or past the range) from the chunk's first
  // channel of image 0 (the input holds fewer than 2^29 elements)
  uint32_t boff[TN][KHW];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + 16 * j + li;
    const bool ok = col < p.N;
    const int cc = ok ? col : 0;
    const int img = cc / p.OHW;
    const int pix = cc - img * p.OHW;
    const int oy = pix / p.OW, ox = pix - oy * p.OW;
    const int iy0 = oy * p.sH - p.pT, ix0 = ox * p.sW - p.pL;
#pragma unroll
    for (int ky = 0; ky < KH; ++ky)
#pragma unroll
      for (int kx = 0; kx < KW; ++kx) {
        const int iy = iy0 + ky * p.dH, ix = ix0 + kx * p.dW;
        const bool in = ok && (unsigned)iy < (unsigned)p.H && (unsigned)ix < (unsigned)p.W;
        boff[j][ky * KW + kx] =
            in ? (uint32_t)(4 * (img * p.x_img + lg * p.HW + iy * p.W + ix)) : kOutside;
      }
  }
  const float *xg = p.B + tc.g * p.x_grp;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float ra[D][TM][KHW], rb[D][TN][KHW];

  auto load = [&](int c, auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int c0 = 4 * c;  // the chunk's first channel
    // weights: the lane's channel c0 + lg exists, else past the range
    const __amdgpu_buffer_rsrc_t ra_rs = buffer_at(abase + c0 * KHW, kRange);
    const bool chok = c0 + lg < cin_g;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // (kOutside + 4 e stays past the range and below 2^32)
      const uint32_t o = chok ? aoff[i] : kOutside;
      if constexpr (KHW % 3 == 0) {
#pragma unroll
        for (int e = 0; e < KHW; e += 3) load3(ra_rs, o + 4 * e, &ra[S][i][e]);
      } else {
#pragma unroll
        for (int e = 0; e < KHW; ++e) ra[S][i][e] = load1(ra_rs, o + 4 * e);
      }
    }
    // input: a lane whose channel lies past the group's last reads +0
    const __amdgpu_buffer_rsrc_t rs = buffer_at(xg + (int64_t)c0 * p.HW, kRange);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < KHW; ++e) rb[S][j][e] = load1(rs, chok ? boff[j][e] : kOutside);
  };
  auto compute = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
#pragma unroll
    for (int e = 0; e < KHW; ++e)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[S][i][e], rb[S][j][e], acc[i][j], 0, 0, 0);
  };
  const int n = ce - cb;
  if (n > 0) {
    const int last = ce - 1;
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) { load(min(cb + (int)decltype(j)::value, last), j); });
    const int full = n - n % D;
    for (int c = 0; c < full; c += D) {
      static_for<D>([&](auto j) __attribute__((always_inline)) {
        constexpr int J = decltype(j)::value;
        load(min(cb + c + J + D - 1, last), std::integral_constant<int, (J + D - 1) % D>{});
        compute(j);
      });
    }
    static_for<D - 1>([&](auto j) __attribute__((always_inline)) {
      if (full + (int)decltype(j)::value < n) compute(j);
    });
  }
  splitk_finish<kBGather, TM, TN, KS>(p, tc.g, m0, n0, wave, acc, red);
}

}  // namespace og
