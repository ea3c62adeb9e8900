// og_launch.hpp -- host-side launchers of libog's kernels: grid shapes and
// the kernel template chosen for a tile variant, mode and operand kind.
// Shared by og_api.hip (argument checks and the choice of variant) and
// og_units.hip (the explicit instantiations of the launchers, one group per
// compilation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "og.h"
#include "og_kernels.hpp"

namespace og::host {

constexpr int64_t kI32Max = 2147483647;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Kernel variants (og_set_variant): 1 VALU 64x64 tile; 2..5 matrix core with
// (bm, bn) output tiles; 6..9 the lane kernel with R = 1, 2, 4, 8 rows per
// wave and 4 waves (so bm = 4R, bn = 64).
struct Tile {
  int variant, bm, bn;
  int per_wave;  // matrix core: 32x64 blocks per wave; lane kernel: rows per wave
};
// 10..13 the chain kernel: (bn columns, compute waves, rows per lane) =
// (64, 4, 1), (64, 2, 1), (16, 1, 1) and (64, 2, 2); its 3x3 convolution
// form of variant 12 has 32 columns.
// 14..16 the chain kernel with matrix-core chains of 4 rows x 64 columns:
// (compute waves, chains per wave) = (4, 1), (2, 2), (2, 1).
// 17 the matrix-core kernel with 256x256 tiles and eight waves.
// 20 the matrix-core kernel with 64x64 tiles of four waves of 16 x 64 outputs
// (v_mfma_f32_16x16x1_4b_f32), both modes.
inline constexpr Tile kTiles[] = {{1, 64, 64, 0},  {2, 128, 256, 4}, {3, 128, 128, 2}, {4, 64, 128, 1},
                           {5, 32, 256, 1}, {6, 4, 64, 1},    {7, 8, 64, 2},    {8, 16, 64, 4},
                           {9, 32, 64, 8},  {10, 4, 64, 1},   {11, 2, 64, 1},   {12, 4, 16, 1},
                           {13, 4, 64, 2},  {14, 16, 64, 1},  {15, 16, 64, 2},  {16, 8, 64, 1},
                           {17, 256, 256, 4}, {20, 64, 64, 1}};
constexpr int kNumVariants = 20;
// 18 the depthwise kernel (Cin/G = 1, any multiplier): the automatic choice
// for those shapes; forced on any other shape it runs the automatic choice.
constexpr int kDepthwiseVariant = 18;
// 19 the grouped direct kernel (grouped 3x3 convolutions with 2 <= Cin/G <= 64
// and Cout/G <= 8): the automatic choice for those shapes; forced on any
// other shape it runs the automatic choice.
constexpr int kGroupedVariant = 19;

inline const Tile &tile_for_variant(int v) {
  for (const Tile &t : kTiles)
    if (t.variant == v) return t;
  return kTiles[1];
}

inline bool is_lane(const Tile &t) { return t.variant >= 6 && t.variant <= 9; }
inline bool is_chain(const Tile &t) { return t.variant >= 10 && t.variant <= 16; }

// Lane variants of a 3x3 or a 1x1 (strided or padded) convolution run the
// lane kernel specialised for that kernel size; its column tiles are 64
// output pixels of one image.
template <int MODE, int KH, int KW>
void launch_lane_conv(int variant, og::Problem p, hipStream_t s) {
  const int tpi = (int)ceil_div(p.OHW, 64);
  const int rpb = 4 * (variant == 6 ? 1 : variant == 7 ? 2 : variant == 8 ? 4 : 8);
  p.tiles_m = (int)ceil_div(p.M, rpb);
  p.tiles_n = (p.N / p.OHW) * tpi;
  const unsigned blocks = (unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups;
  const dim3 grid(blocks), block(256);
  switch (variant) {
    case 6: hipLaunchKernelGGL((og::lane_conv_kernel<MODE, KH, KW, 1, 4, 2>), grid, block, 0, s, p); break;
    case 7: hipLaunchKernelGGL((og::lane_conv_kernel<MODE, KH, KW, 2, 4, 2>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((og::lane_conv_kernel<MODE, KH, KW, 4, 4, 2>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((og::lane_conv_kernel<MODE, KH, KW, 8, 4, 2>), grid, block, 0, s, p); break;
  }
}

// The chain kernel of variant v for a matrix product (CONV false; VEC: B
// rows 16-byte aligned, read 16 bytes per load) or a KH x KW convolution; its
// column tiles of a convolution are BN pixels of one image.
template <int MODE, bool CONV, int LD, int KH, int KW>
void launch_chain(int v, og::Problem p, hipStream_t s) {
  // Exact mode of the matrix-core chains (14..16) runs the DPP chains of
  // the same block shape (10, 13, 11): its products made on the matrix
  // cores would still need a VALU add each, and the compiler cannot keep
  // their independent products from piling up in registers.
  if (MODE == og::kExact && v >= 14) v = v == 14 ? 10 : v == 15 ? 13 : 11;
  const bool mf = v >= 14;
  const int bn = v == 12 ? (KH * KW == 1 ? 16 : 32) : 64;
  const int cw = v == 10 || v == 14 ? 4 : v == 12 ? 1 : 2;  // compute waves
  const int rows = mf ? cw * 4 * (v == 15 ? 2 : 1) : cw * (64 / bn) * (v == 13 ? 2 : 1);
  const int pw = 4 * bn / 64;  // B producer waves (and one weight wave)
  p.tiles_m = (int)ceil_div(p.M, rows);
  p.tiles_n = CONV ? (int)((p.N / p.OHW) * ceil_div(p.OHW, bn)) : (int)ceil_div(p.N, bn);
  const unsigned blocks = (unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups;
  const dim3 grid(blocks), block(64 * (cw + pw + 1));
  switch (v) {
    case 10: hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 4, 1, false>), grid, block, 0, s, p); break;
    case 11: hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 2, 1, false>), grid, block, 0, s, p); break;
    case 12:
      if constexpr (KH * KW == 1)
        hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 16, 1, 1, false>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 32, 1, 1, false>), grid, block, 0, s, p);
      break;
    case 13: hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 2, 2, false>), grid, block, 0, s, p); break;
    default:
      if constexpr (MODE == og::kFast) {
        if (v == 14)
          hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 4, 1, true>), grid, block, 0, s, p);
        else if (v == 15)
          hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 2, 2, true>), grid, block, 0, s, p);
        else
          hipLaunchKernelGGL((og::chain_kernel<MODE, CONV, LD, KH, KW, 64, 2, 1, true>), grid, block, 0, s, p);
      }
      break;
  }
}

// The chain kernel of a 3x3 or 1x1 convolution (false for other windows).
template <int MODE>
bool launch_conv_chain(int v, og::Problem p, hipStream_t s) {
  if (p.KH == 3 && p.KW == 3) {
    // a kernel row's three taps in one load: horizontal dilation 1, the
    // row at least 3 wide, left and right pads at most 1
    if (p.dW == 1 && p.W >= 3 && p.pL <= 1 && p.pR <= 1)
      launch_chain<MODE, true, og::kLdRow3, 3, 3>(v, p, s);
    else
      launch_chain<MODE, true, og::kLdTap, 3, 3>(v, p, s);
    return true;
  }
  if (p.KH == 1 && p.KW == 1) {
    launch_chain<MODE, true, og::kLdTap, 1, 1>(v, p, s);
    return true;
  }
  return false;
}

// The lane kernel of a gathered 3x3 or 1x1 convolution (false for other windows).
template <int MODE>
bool launch_lane_conv_any(int v, og::Problem p, hipStream_t s) {
  if (p.KH == 3 && p.KW == 3) {
    launch_lane_conv<MODE, 3, 3>(v, p, s);
    return true;
  }
  if (p.KH == 1 && p.KW == 1) {
    launch_lane_conv<MODE, 1, 1>(v, p, s);
    return true;
  }
  return false;
}

// D: register-ring depth of the staged loads (chunks in flight).
template <int MODE, int KIND, bool AV, bool BV>
void launch_tile(const Tile &t, og::Problem p, hipStream_t s) {
  if (is_chain(t)) {
    if constexpr (KIND == og::kBMatrix) {
      if (BV) return launch_chain<MODE, false, og::kLdVec, 1, 1>(t.variant, p, s);
      return launch_chain<MODE, false, og::kLdTap, 1, 1>(t.variant, p, s);
    } else {
      if (launch_conv_chain<MODE>(t.variant, p, s)) return;
      // other window sizes: the lane kernel with one row per wave
      return launch_tile<MODE, KIND, AV, BV>(tile_for_variant(6), p, s);
    }
  }
  if constexpr (KIND == og::kBGather) {
    if (is_lane(t) && launch_lane_conv_any<MODE>(t.variant, p, s)) return;
  }
  // Exact mode keeps two k steps of products beside the accumulators: with
  // two 32x64 blocks per wave (128x256, 128x128 and 256x256 tiles) that no
  // longer fits the registers of two waves per SIMD, so variants 2, 3 and 17
  // run 64x128 tiles.  With gathered B it keeps one product and runs 128x128
  // tiles.
  const bool big = t.variant == 2 || t.variant == 3 || t.variant == 17;
  const Tile &tt = (MODE == og::kExact && big) ? tile_for_variant(KIND == og::kBGather ? 3 : 4) : t;
  p.tiles_m = (int)ceil_div(p.M, tt.bm);
  p.tiles_n = (int)ceil_div(p.N, tt.bn);
  const unsigned blocks = (unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups;
  const dim3 grid(blocks), block(256);
  if constexpr (MODE == og::kExact) {
    if (big) {
      if constexpr (KIND == og::kBGather)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 128, 128, 2, 2, KIND, AV, BV, 2>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 128, 2, 2, KIND, AV, BV, 4>), grid, block, 0, s, p);
      return;
    }
  }
  switch (t.variant) {
    case 1: hipLaunchKernelGGL((og::valu_kernel<MODE, KIND>), grid, block, 0, s, p); break;
    case 2:
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 128, 256, 2, 2, KIND, AV, BV, 2>), grid, block, 0, s, p);
      break;
    case 3:
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 128, 128, 2, 2, KIND, AV, BV, 2>), grid, block, 0, s, p);
      break;
    case 4: hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 128, 2, 2, KIND, AV, BV, 4>), grid, block, 0, s, p); break;
    case 5: hipLaunchKernelGGL((og::mfma_kernel<MODE, 32, 256, 1, 4, KIND, AV, BV, 2>), grid, block, 0, s, p); break;
    case 17:  // eight waves: the B tile (and its gather) serves 256 rows
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 256, 256, 4, 2, KIND, AV, BV, 2>), grid, dim3(512), 0, s, p);
      break;
    case 20:  // four waves of 16 x 64 outputs
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 64, 4, 1, KIND, AV, BV, 2, 16>), grid, block, 0, s, p);
      break;
    // (rings of two chunks: deeper rings cost more in occupancy than they
    // gain in hidden latency, measured on the ResNet-50 layers and products)
    case 6: hipLaunchKernelGGL((og::lane_kernel<MODE, KIND, 1, 4, 2>), grid, block, 0, s, p); break;
    case 7: hipLaunchKernelGGL((og::lane_kernel<MODE, KIND, 2, 4, 2>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((og::lane_kernel<MODE, KIND, 4, 4, 2>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((og::lane_kernel<MODE, KIND, 8, 4, 2>), grid, block, 0, s, p); break;
  }
}

// AV / BV: 16-byte loads of A rows / B rows (every address and every
// row length a multiple of 16 bytes, so no load crosses the end of a row).
template <int MODE, int KIND>
void launch_vec(bool av, bool bv, const Tile &t, const og::Problem &p, hipStream_t s) {
  if (av && bv)
    launch_tile<MODE, KIND, true, true>(t, p, s);
  else if (av)
    launch_tile<MODE, KIND, true, false>(t, p, s);
  else if (bv)
    launch_tile<MODE, KIND, false, true>(t, p, s);
  else
    launch_tile<MODE, KIND, false, false>(t, p, s);
}

inline bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15) == 0; }

template <int MODE, bool EPI, int KH, int KW>
void launch_dw_window(og::Problem p, int per_lane, dim3 grid, hipStream_t s) {
  if (per_lane == 4)
    hipLaunchKernelGGL((og::dw_kernel<MODE, KH, KW, 4, EPI>), grid, dim3(256), 0, s, p);
  else if (per_lane == 2)
    hipLaunchKernelGGL((og::dw_kernel<MODE, KH, KW, 2, EPI>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((og::dw_kernel<MODE, KH, KW, 1, EPI>), grid, dim3(256), 0, s, p);
}

// The band form of the depthwise kernel (input rows staged in LDS) for
// strided or 5x5 windows on planes at least 28 pixels wide: bands of at
// most 1024 outputs, enough bands for at least 1024 blocks, every band at
// least 128 outputs, the staged rows within 32 KB.  Returns false (and
// launches nothing) where the shape does not qualify.
template <int MODE, bool EPI>
bool launch_dw_band(og::Problem p, int64_t planes, int64_t OH, int64_t OW, hipStream_t s) {
  const bool w3 = p.KH == 3 && p.KW == 3, w5 = p.KH == 5 && p.KW == 5;
  if (!(w3 || w5) || (w3 && p.sH == 1 && p.sW == 1) || OW < 28) return false;
  const int64_t iw = (OW - 1) * p.sW + (int64_t)(p.KW - 1) * p.dW + 1;
  int64_t nb = std::max(ceil_div(OH * OW, 1024), ceil_div(1024, planes));
  nb = std::min(nb, OH);
  const int64_t bh = ceil_div(OH, nb);
  nb = ceil_div(OH, bh);
  const int64_t ih = (bh - 1) * p.sH + (int64_t)(p.KH - 1) * p.dH + 1;
  if (planes * nb < 1024 || bh * OW < 128 || ih * iw > 8192 || planes * nb > kI32Max) return false;
  p.bh = (int)bh;
  p.ih = (int)ih;
  p.iw = (int)iw;
  p.tiles_m = (int)nb;
  p.tiles_n = (int)planes;
  const dim3 grid((unsigned)(planes * nb)), block(256);
  const size_t lds = (size_t)(4 * ih * iw);
  if (w3)
    hipLaunchKernelGGL((og::dw_band_kernel<MODE, 3, 3, EPI>), grid, block, lds, s, p);
  else
    hipLaunchKernelGGL((og::dw_band_kernel<MODE, 5, 5, EPI>), grid, block, lds, s, p);
  return true;
}

// The grouped direct kernel, R = Cout/G rounded up to 1, 2, 4 or 8 rows per lane.
template <int MODE, bool EPI>
void launch_grouped_mode(og::Problem p, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div((int64_t)p.tiles_m * p.tiles_n, 4)), block(256);
  if (p.M <= 1)
    hipLaunchKernelGGL((og::grouped_kernel<MODE, 3, 3, 1, EPI>), grid, block, 0, s, p);
  else if (p.M <= 2)
    hipLaunchKernelGGL((og::grouped_kernel<MODE, 3, 3, 2, EPI>), grid, block, 0, s, p);
  else if (p.M <= 4)
    hipLaunchKernelGGL((og::grouped_kernel<MODE, 3, 3, 4, EPI>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((og::grouped_kernel<MODE, 3, 3, 8, EPI>), grid, block, 0, s, p);
}

template <int MODE, bool EPI>
void launch_dw(og::Problem p, int per_lane, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div((int64_t)p.tiles_m * p.tiles_n, 4));
  if (p.KH == 3 && p.KW == 3)
    launch_dw_window<MODE, EPI, 3, 3>(p, per_lane, grid, s);
  else if (p.KH == 5 && p.KW == 5)  // one output per lane (dw_outputs_per_lane)
    hipLaunchKernelGGL((og::dw_kernel<MODE, 5, 5, 1, EPI>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((og::dw_kernel<MODE, 0, 0, 1, EPI>), grid, dim3(256), 0, s, p);
}

// The depthwise and grouped direct kernels are compiled with and without the
// epilogue (EPI): (mode, epilogue) -> one of four instantiations.
template <template <int, bool> class L, class... A>
auto by_mode_epi(int mode, bool epi, A &&...a) {
  if (mode == OG_MODE_EXACT)
    return epi ? L<og::kExact, true>::run(a...) : L<og::kExact, false>::run(a...);
  return epi ? L<og::kFast, true>::run(a...) : L<og::kFast, false>::run(a...);
}
// (The run members are defined outside their classes: defined inside they
// would be inline, and an extern template declaration does not keep inline
// members, and the kernels they launch, from being instantiated.)
template <int MODE, bool EPI>
struct DwBand {
  static bool run(og::Problem p, int64_t planes, int64_t OH, int64_t OW, hipStream_t s);
};
template <int MODE, bool EPI>
bool DwBand<MODE, EPI>::run(og::Problem p, int64_t planes, int64_t OH, int64_t OW,
                            hipStream_t s) {
  return launch_dw_band<MODE, EPI>(p, planes, OH, OW, s);
}
template <int MODE, bool EPI>
struct Dw {
  static int run(og::Problem p, int per_lane, hipStream_t s);
};
template <int MODE, bool EPI>
int Dw<MODE, EPI>::run(og::Problem p, int per_lane, hipStream_t s) {
  launch_dw<MODE, EPI>(p, per_lane, s);
  return 0;
}
template <int MODE, bool EPI>
struct Grouped {
  static int run(og::Problem p, hipStream_t s);
};
template <int MODE, bool EPI>
int Grouped<MODE, EPI>::run(og::Problem p, hipStream_t s) {
  launch_grouped_mode<MODE, EPI>(p, s);
  return 0;
}

// The row-dot kernel (single-column products): one wave of 64 rows per
// block, a ring of 8 chunks of 16 taps; VEC: 16-byte loads of the rows.
template <int MODE>
void launch_rowdot_mode(og::Problem p, bool vec, hipStream_t s) {
  p.tiles_m = (int)ceil_div(p.M, 64);
  p.tiles_n = 1;
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.groups), block(64);
  if (vec)
    hipLaunchKernelGGL((og::rowdot_kernel<MODE, true, 8>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((og::rowdot_kernel<MODE, false, 8>), grid, block, 0, s, p);
}

// One row against the rows of an N x K matrix (k-contiguous, 16-byte
// aligned, k a multiple of 4) on the chain kernel in its single-row form
// (variant 12's shape: blocks of 16 columns, one compute wave of 4 lane rows,
// one producer wave, one weight wave): the N x K operand streamed once
// through LDS, 16 bytes of one column per load and no transpose.
// p: A = the row (M = 1), B = the N x K operand (ldb its row stride), C = the
// n outputs (contiguous), N = n, K = k.
template <int MODE, int BN, int CW, int R, bool MF>
void launch_chain_vt_shape(og::Problem p, hipStream_t s) {
  constexpr int ROWS = og::chain_rows(CW, BN, R, MF);
  using CS = og::ChainShape<1, BN, ROWS>;
  p.tiles_m = (int)ceil_div(p.M, ROWS);
  p.tiles_n = (int)ceil_div(p.N, BN);
  p.groups = 1;
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n), block(64 * (CW + CS::PW + 1));
  hipLaunchKernelGGL((og::chain_kernel<MODE, false, og::kLdVecT, 1, 1, BN, CW, R, MF>), grid,
                     block, 0, s, p);
}

// More than 16 rows in fast mode: the matrix-core chains of variant 14's
// shape (16 rows x 64 columns per block, the N x K operand streamed once per
// 16 rows instead of once per 4).
template <int MODE>
void launch_chain_vt_mode(og::Problem p, hipStream_t s) {
  if constexpr (MODE == og::kFast) {
    if (p.M > 16) return launch_chain_vt_shape<MODE, 64, 4, 1, true>(p, s);
  }
  launch_chain_vt_shape<MODE, 16, 1, 1, false>(p, s);
}

// The product with a transposed B (N x K) runs the tile kernels that stage B
// like A: the VALU kernel (variant 1) and the matrix-core kernel (2..5, 17,
// 20, with exact mode's 64x128 tiles for 2, 3 and 17).
template <int MODE, bool AV, bool BV>
void launch_nt_tile(const Tile &t, og::Problem p, hipStream_t s) {
  constexpr int K = og::kBMatrixT;
  const bool big = t.variant == 2 || t.variant == 3 || t.variant == 17;
  const Tile &tt = (MODE == og::kExact && big) ? tile_for_variant(4) : t;
  p.tiles_m = (int)ceil_div(p.M, tt.bm);
  p.tiles_n = (int)ceil_div(p.N, tt.bn);
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n), block(256);
  if (MODE == og::kExact && big) {
    hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 128, 2, 2, K, AV, BV, 4>), grid, block, 0, s, p);
    return;
  }
  switch (tt.variant) {
    case 1: hipLaunchKernelGGL((og::valu_kernel<MODE, K>), grid, block, 0, s, p); break;
    case 2:
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 128, 256, 2, 2, K, AV, BV, 2>), grid, block, 0, s, p);
      break;
    case 3:
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 128, 128, 2, 2, K, AV, BV, 2>), grid, block, 0, s, p);
      break;
    case 5: hipLaunchKernelGGL((og::mfma_kernel<MODE, 32, 256, 1, 4, K, AV, BV, 2>), grid, block, 0, s, p); break;
    case 17:
      if constexpr (MODE == og::kFast)
        hipLaunchKernelGGL((og::mfma_kernel<MODE, 256, 256, 4, 2, K, AV, BV, 2>), grid, dim3(512), 0, s, p);
      break;
    case 20: hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 64, 4, 1, K, AV, BV, 2, 16>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((og::mfma_kernel<MODE, 64, 128, 2, 2, K, AV, BV, 4>), grid, block, 0, s, p); break;
  }
}

template <int MODE>
void launch_nt(bool av, bool bv, const Tile &t, const og::Problem &p, hipStream_t s) {
  if (av && bv)
    launch_nt_tile<MODE, true, true>(t, p, s);
  else if (av)
    launch_nt_tile<MODE, true, false>(t, p, s);
  else if (bv)
    launch_nt_tile<MODE, false, true>(t, p, s);
  else
    launch_nt_tile<MODE, false, false>(t, p, s);
}

// ---------------------------------------------------------------------------
// Split-k kernels (OG_MODE_FAST_MFMA): variant -> (16 TM) x (16 TN) output
// tiles with KS waves sharing k.
// ---------------------------------------------------------------------------
struct SplitTile {
  int variant, tm, tn, ks;
};
inline constexpr SplitTile kSplitTiles[] = {
    {21, 1, 1, 16}, {22, 1, 2, 8}, {23, 2, 2, 8}, {24, 2, 4, 4}, {25, 2, 2, 4}};
constexpr int kFirstSplitVariant = 21, kLastSplitVariant = 25;
inline bool is_split(int v) { return v >= kFirstSplitVariant && v <= kLastSplitVariant; }

inline const SplitTile &split_tile(int v) {
  for (const SplitTile &t : kSplitTiles)
    if (t.variant == v) return t;
  return kSplitTiles[0];
}

template <int KIND, bool AV, bool BV, int KH, int KW>
void launch_splitk(int variant, og::Problem p, hipStream_t s) {
  const SplitTile &t = split_tile(variant);
  p.tiles_m = (int)ceil_div(p.M, 16 * t.tm);
  p.tiles_n = (int)ceil_div(p.N, 16 * t.tn);
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups),
      block(64 * t.ks);
  if constexpr (KIND == og::kBGather && KH * KW > 1) {
    // a window known at compile time: chunks of four channels by the window
    switch (t.variant) {
      case 21: hipLaunchKernelGGL((og::splitk_conv_kernel<AV, 1, 1, 16, KH, KW>), grid, block, 0, s, p); break;
      case 22: hipLaunchKernelGGL((og::splitk_conv_kernel<AV, 1, 2, 8, KH, KW>), grid, block, 0, s, p); break;
      case 23: hipLaunchKernelGGL((og::splitk_conv_kernel<AV, 2, 2, 8, KH, KW>), grid, block, 0, s, p); break;
      case 24: hipLaunchKernelGGL((og::splitk_conv_kernel<AV, 2, 4, 4, KH, KW>), grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL((og::splitk_conv_kernel<AV, 2, 2, 4, KH, KW>), grid, block, 0, s, p); break;
    }
    return;
  }
  switch (t.variant) {
    case 21: hipLaunchKernelGGL((og::splitk_kernel<KIND, AV, BV, 1, 1, 16, KH, KW>), grid, block, 0, s, p); break;
    case 22: hipLaunchKernelGGL((og::splitk_kernel<KIND, AV, BV, 1, 2, 8, KH, KW>), grid, block, 0, s, p); break;
    case 23: hipLaunchKernelGGL((og::splitk_kernel<KIND, AV, BV, 2, 2, 8, KH, KW>), grid, block, 0, s, p); break;
    case 24: hipLaunchKernelGGL((og::splitk_kernel<KIND, AV, BV, 2, 4, 4, KH, KW>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((og::splitk_kernel<KIND, AV, BV, 2, 2, 4, KH, KW>), grid, block, 0, s, p); break;
  }
}

// Matrix products: B row-major (bt false) or given as its transpose (bt);
// av / bv: 16-byte loads of A rows / of the transposed B's rows.
// (Instantiated in og_units.hip.)
void launch_splitk_matrix(int variant, bool av, bool bv, bool bt, const og::Problem &p,
                          hipStream_t s);
// Convolutions: input planes read in place (1x1, stride 1, no padding) or
// gathered (3x3 and 1x1 windows compiled in, others read at run time).
void launch_splitk_conv(int variant, bool av, bool planes, const og::Problem &p, hipStream_t s);

// ---------------------------------------------------------------------------
// Halo kernel (3x3 windows) over 64 lanes of one image.  Matrix-core
// chains: variant 26 four waves of one chain of 4 output channels (16 rows
// per block), 27 four waves of two chains (32 rows), 28 eight waves of one
// chain (32 rows, two waves per SIMD).  DPP steps (a lane's own rows, the
// weights broadcast within rows of 16 lanes; for latency-bound shapes):
// variant 31 four waves of one row (4 rows per block), 32 eight waves of one
// row (8 rows), 33 four waves of two rows (8 rows).
// ---------------------------------------------------------------------------
constexpr int kFirstHaloVariant = 26, kLastHaloVariant = 28;
constexpr int kFirstHaloDppVariant = 31, kLastHaloDppVariant = 33;
inline bool is_halo(int v) {
  return (v >= kFirstHaloVariant && v <= kLastHaloVariant) ||
         (v >= kFirstHaloDppVariant && v <= kLastHaloDppVariant);
}
// shape of a halo variant: rows per chain set R, waves CW, DPP steps
struct HaloShape {
  int r, cw;
  bool dpp;
};
inline HaloShape halo_shape(int v) {
  switch (v) {
    case 26: return {1, 4, false};
    case 27: return {2, 4, false};
    case 28: return {1, 8, false};
    case 31: return {1, 4, true};
    case 32: return {1, 8, true};
    default: return {2, 4, true};
  }
}
// output rows per block
inline int halo_block_rows(int v) {
  const HaloShape h = halo_shape(v);
  return (h.dpp ? 1 : 4) * h.r * h.cw;
}

// The staging of a shape: rows a tile of 64 output pixels stages (the
// output rows 64 consecutive pixels can touch, then the rows their windows
// reach, padding rows included), halo loads per lane and channel (ni) and
// their width (16 bytes when every staged input row starts 16-byte
// aligned), the dynamic LDS: three buffers of 16 channels of rows x padded
// width positions, then three weight stages of each wave's rows x 144 taps.
// Horizontal dilation 1 and weight rows of whole 16-byte quads (Cin/G a
// multiple of 4) only.
struct HaloPlan {
  int rows, ni;
  bool hv;
  int vpitch;       // stride 1: the lanes' rows of cells, as wide as the padded input row; else 0
  int64_t tiles;    // tiles of 64 lanes per image
  int64_t buf_lds;  // bytes of one halo buffer
};
// a wave's weight stage in floats (its rows of 144 taps -- 4 * R on the
// matrix cores, R with DPP steps -- padded to whole loads of 64 lanes x 16
// bytes), the weight stages of a block of variant v in bytes (two per wave),
// and the LDS a workgroup may hold on gfx950
constexpr int64_t halo_weight_stage(int R, bool dpp) { return ((dpp ? 1 : 4) * R * 144 / 4 + 63) / 64 * 64 * 4; }
inline int64_t halo_weight_lds(int v) {
  const HaloShape h = halo_shape(v);
  return (int64_t)h.cw * 2 * halo_weight_stage(h.r, h.dpp) * 4;
}
constexpr int64_t kHaloMaxLds = 160 * 1024;
inline bool halo_plan(const og::Problem &p, bool x_aligned16, HaloPlan &h) {
  if (p.dW != 1 || !p.a_vec) return false;
  const int oh = p.OHW / p.OW;
  // at stride 1 the lanes take cells of rows as wide as the padded input row
  // (a tile's lanes past the image included); else 64 consecutive pixels
  h.vpitch = p.sH == 1 && p.sW == 1 ? p.W + p.pL + p.pR : 0;
  const int64_t vw = h.vpitch > 0 ? h.vpitch : p.OW, ncell = (int64_t)oh * vw;
  h.tiles = ceil_div(ncell, 64);
  // the most rows of cells a tile's lanes span
  int64_t orows = 1;
  for (int64_t t = 0; t < h.tiles; ++t) {
    const int64_t lastc = h.vpitch > 0 ? 64 * t + 63 : std::min(64 * t + 63, ncell - 1);
    orows = std::max(orows, lastc / vw - 64 * t / vw + 1);
  }
  h.rows = (int)((orows - 1) * p.sH + (p.KH - 1) * p.dH + 1);
  const int64_t hlen = (int64_t)std::min(h.rows, p.H) * p.W;  // input floats of a channel
  h.hv = x_aligned16 && p.W % 4 == 0 && p.HW % 4 == 0 && p.x_img % 4 == 0 && p.x_grp % 4 == 0;
  if (h.hv)
    h.ni = hlen <= 256 ? 1 : hlen <= 512 ? 2 : 0;
  else
    h.ni = hlen <= 128 ? 2 : hlen <= 256 ? 4 : hlen <= 512 ? 8 : 0;
  // a buffer: rows * (W + pL + pR) + 3 cells of 20 floats (16 channels and
  // 4 of padding)
  h.buf_lds = ((int64_t)h.rows * (p.W + p.pL + p.pR) + 3) * 20 * 4;
  return h.ni != 0 && 2 * h.buf_lds + halo_weight_lds(26) <= kHaloMaxLds;
}
// whether variant v's block (two halo buffers and its weight stages) fits the LDS
inline bool halo_fits(const HaloPlan &h, int v) { return 2 * h.buf_lds + halo_weight_lds(v) <= kHaloMaxLds; }

template <int MODE, int R, int CW, bool DPP, int NI, bool HV, bool AV, int NBUF>
void launch_halo_nbuf(const og::Problem &p, const HaloPlan &h, hipStream_t s) {
  constexpr int NWS = 2;
  const auto kernel = og::halo_kernel<MODE, 3, 3, R, CW, NI, HV, AV, NWS, NBUF, DPP>;
  // more than 64 KB of dynamic LDS must be allowed per kernel, once
  static const hipError_t allowed =
      hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHaloMaxLds);
  (void)allowed;
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups), block(64 * CW);
  const size_t lds = (size_t)(NBUF * h.buf_lds) + (size_t)CW * NWS * halo_weight_stage(R, DPP) * 4;
  hipLaunchKernelGGL(kernel, grid, block, lds, s, p);
}

// Two weight stages per wave (measured over 80 3x3 convolutions, three
// stages, which hide more of the weight loads' latency, took 2 % more time
// in all, the LDS they hold costing blocks per compute unit); three halo
// buffers where they fit and the launch's blocks need no more compute-unit
// slots than three buffers leave (the kernels use over 128 registers: at
// most two waves per SIMD), else two (a second barrier per chunk).
template <int MODE, int R, int CW, bool DPP, int NI, bool HV, bool AV>
void launch_halo_shape(og::Problem p, const HaloPlan &h, hipStream_t s) {
  p.hrows = h.rows;
  p.vpitch = h.vpitch;
  p.tiles_m = (int)ceil_div(p.M, (DPP ? 1 : 4) * R * CW);
  p.tiles_n = (int)((p.N / p.OHW) * h.tiles);
  auto per_cu = [&](int nbuf) {
    const int64_t lds = nbuf * h.buf_lds + (int64_t)CW * 2 * halo_weight_stage(R, DPP) * 4;
    return lds > kHaloMaxLds ? 0 : std::min<int64_t>(kHaloMaxLds / lds, 8 / CW);
  };
  const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n * p.groups;
  if (per_cu(3) > 0 && (per_cu(3) >= per_cu(2) || blocks <= 256 * per_cu(3)))
    return launch_halo_nbuf<MODE, R, CW, DPP, NI, HV, AV, 3>(p, h, s);
  launch_halo_nbuf<MODE, R, CW, DPP, NI, HV, AV, 2>(p, h, s);
}

template <int MODE, int R, int CW, bool DPP>
void launch_halo_r(og::Problem p, const HaloPlan &h, hipStream_t s) {
  if (h.hv) {
    if (h.ni == 1) return launch_halo_shape<MODE, R, CW, DPP, 1, true, true>(p, h, s);
    return launch_halo_shape<MODE, R, CW, DPP, 2, true, true>(p, h, s);
  }
  if (h.ni == 2) return launch_halo_shape<MODE, R, CW, DPP, 2, false, true>(p, h, s);
  if (h.ni == 4) return launch_halo_shape<MODE, R, CW, DPP, 4, false, true>(p, h, s);
  return launch_halo_shape<MODE, R, CW, DPP, 8, false, true>(p, h, s);
}

// A 3x3 convolution (gathered B) on a halo variant (26..28, 31..33),
// planned by halo_plan, in exact (0) or fast (1) mode.
void launch_halo_conv(int variant, int mode, const og::Problem &p, const HaloPlan &h, hipStream_t s);
// (its kernels by group: matrix-core fast, matrix-core exact, DPP both modes)
void launch_halo_exact(int variant, const og::Problem &p, const HaloPlan &h, hipStream_t s);
void launch_halo_dpp(int variant, int mode, const og::Problem &p, const HaloPlan &h, hipStream_t s);

// ---------------------------------------------------------------------------
// Panel kernel (fast mode: 1x1 convolutions, any stride and padding, and
// matrix products): four waves over 64 columns, variant 29 one chain of 4
// rows per wave (16 rows per block) in chunks of 64 steps and four stages
// (96 KB of LDS), 30 two chains (32 rows) in chunks of 32 steps and five
// stages (60 KB, two blocks per compute unit).  B rows are read 16 bytes
// per lane (bv) where every row of the panel starts 16-byte aligned and the
// column count is a multiple of 4.
// ---------------------------------------------------------------------------
constexpr int kFirstPanelVariant = 29, kLastPanelVariant = 30;
inline bool is_panel(int v) { return v >= kFirstPanelVariant && v <= kLastPanelVariant; }

template <int KIND, int R, bool BV, bool AV>
void launch_panel_shape(og::Problem p, hipStream_t s) {
  constexpr int CW = 4, CC = R == 1 ? 64 : 32, NS = R == 1 ? 4 : 5;
  const auto kernel = og::panel_kernel<KIND, R, CW, CC, NS, BV, AV>;
  p.tiles_m = (int)ceil_div(p.M, 4 * R * CW);
  p.tiles_n = KIND == og::kBMatrix ? (int)ceil_div(p.N, 64) : (int)((p.N / p.OHW) * ceil_div(p.OHW, 64));
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)p.groups), block(64 * CW);
  const size_t lds = (size_t)(NS * CC * 64 + CW * NS * 4 * R * CC) * 4;  // B stages, weight stages
  // more than 64 KB of dynamic LDS must be allowed per kernel, once
  static const hipError_t allowed =
      hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)allowed;
  hipLaunchKernelGGL(kernel, grid, block, lds, s, p);
}

// A matrix product (kind kBMatrix) or a 1x1 convolution (kBPlanes, kBGather)
// on variant 29 or 30.
void launch_panel(int variant, int kind, bool bv, bool av, const og::Problem &p, hipStream_t s);

// Entry points of the kernel groups, each instantiated in one compilation
// of og_units.hip (so the groups compile in parallel) and declared extern
// here so no other unit instantiates them.
template <int MODE, int KIND>
void launch_kind(bool av, bool bv, const Tile &t, const og::Problem &p, hipStream_t s) {
  launch_vec<MODE, KIND>(av, bv, t, p, s);
}

#define OG_MODES_KINDS(X)                                                              \
  X(og::kExact, og::kBMatrix) X(og::kFast, og::kBMatrix) X(og::kExact, og::kBGather) \
      X(og::kFast, og::kBGather) X(og::kExact, og::kBPlanes) X(og::kFast, og::kBPlanes)
#define OG_EXTERN_KIND(M, K) \
  extern template void launch_kind<M, K>(bool, bool, const Tile &, const og::Problem &, hipStream_t);
OG_MODES_KINDS(OG_EXTERN_KIND)
#undef OG_EXTERN_KIND
#define OG_EXTERN_MODE(M)                                                                     \
  extern template bool launch_conv_chain<M>(int, og::Problem, hipStream_t);                  \
  extern template bool launch_lane_conv_any<M>(int, og::Problem, hipStream_t);               \
  extern template void launch_nt<M>(bool, bool, const Tile &, const og::Problem &, hipStream_t); \
  extern template void launch_chain_vt_mode<M>(og::Problem, hipStream_t);                    \
  extern template void launch_rowdot_mode<M>(og::Problem, bool, hipStream_t);                \
  extern template struct DwBand<M, false>;                                                     \
  extern template struct DwBand<M, true>;                                                      \
  extern template struct Dw<M, false>;                                                         \
  extern template struct Dw<M, true>;                                                          \
  extern template struct Grouped<M, false>;                                                    \
  extern template struct Grouped<M, true>;
OG_EXTERN_MODE(og::kExact)
OG_EXTERN_MODE(og::kFast)
#undef OG_EXTERN_MODE


}  // namespace og::host
