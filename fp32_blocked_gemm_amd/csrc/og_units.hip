// og_units.hip -- explicit instantiations of libog's kernel launchers.
//
// The build compiles this file once per group (-DOG_UNIT=1..OG_UNITS), each
// compilation instantiating one group of launchers and so the kernels they
// launch; the groups compile in parallel and link into one library.  Every
// launcher is instantiated in exactly one group (og_launch.hpp declares them
// all extern).
#include "og_launch.hpp"

#ifndef OG_UNIT
#error "compile with -DOG_UNIT=<group>"
#endif

namespace og::host {

#define OG_KIND(M, K) \
  template void launch_kind<M, K>(bool, bool, const Tile &, const og::Problem &, hipStream_t);

#if OG_UNIT == 1
OG_KIND(og::kExact, og::kBMatrix)
#elif OG_UNIT == 2
OG_KIND(og::kFast, og::kBMatrix)
#elif OG_UNIT == 3
OG_KIND(og::kExact, og::kBGather)
template bool launch_lane_conv_any<og::kExact>(int, og::Problem, hipStream_t);
#elif OG_UNIT == 4
OG_KIND(og::kFast, og::kBGather)
template bool launch_lane_conv_any<og::kFast>(int, og::Problem, hipStream_t);
#elif OG_UNIT == 5
OG_KIND(og::kExact, og::kBPlanes)
#elif OG_UNIT == 6
OG_KIND(og::kFast, og::kBPlanes)
#elif OG_UNIT == 7
template bool launch_conv_chain<og::kExact>(int, og::Problem, hipStream_t);
#elif OG_UNIT == 8
template bool launch_conv_chain<og::kFast>(int, og::Problem, hipStream_t);
#elif OG_UNIT == 9
template void launch_nt<og::kExact>(bool, bool, const Tile &, const og::Problem &, hipStream_t);
template void launch_chain_vt_mode<og::kExact>(og::Problem, hipStream_t);
#elif OG_UNIT == 10
template void launch_nt<og::kFast>(bool, bool, const Tile &, const og::Problem &, hipStream_t);
template void launch_chain_vt_mode<og::kFast>(og::Problem, hipStream_t);
#elif OG_UNIT == 11
template void launch_rowdot_mode<og::kExact>(og::Problem, bool, hipStream_t);
template void launch_rowdot_mode<og::kFast>(og::Problem, bool, hipStream_t);
template struct DwBand<og::kExact, false>;
template struct DwBand<og::kExact, true>;
template struct DwBand<og::kFast, false>;
template struct DwBand<og::kFast, true>;
template struct Dw<og::kExact, false>;
template struct Dw<og::kExact, true>;
template struct Dw<og::kFast, false>;
template struct Dw<og::kFast, true>;
template struct Grouped<og::kExact, false>;
template struct Grouped<og::kExact, true>;
template struct Grouped<og::kFast, false>;
template struct Grouped<og::kFast, true>;
#elif OG_UNIT == 12
void launch_splitk_matrix(int variant, bool av, bool bv, bool bt, const og::Problem &p,
                          hipStream_t s) {
  if (bt) {
    if (av && bv) return launch_splitk<og::kBMatrixT, true, true, 0, 0>(variant, p, s);
    if (av) return launch_splitk<og::kBMatrixT, true, false, 0, 0>(variant, p, s);
    if (bv) return launch_splitk<og::kBMatrixT, false, true, 0, 0>(variant, p, s);
    return launch_splitk<og::kBMatrixT, false, false, 0, 0>(variant, p, s);
  }
  if (av) return launch_splitk<og::kBMatrix, true, false, 0, 0>(variant, p, s);
  return launch_splitk<og::kBMatrix, false, false, 0, 0>(variant, p, s);
}
#elif OG_UNIT == 13
void launch_splitk_conv(int variant, bool av, bool planes, const og::Problem &p, hipStream_t s) {
  if (planes) {
    if (av) return launch_splitk<og::kBPlanes, true, false, 0, 0>(variant, p, s);
    return launch_splitk<og::kBPlanes, false, false, 0, 0>(variant, p, s);
  }
  if (p.KH == 3 && p.KW == 3) {
    if (av) return launch_splitk<og::kBGather, true, false, 3, 3>(variant, p, s);
    return launch_splitk<og::kBGather, false, false, 3, 3>(variant, p, s);
  }
  if (p.KH == 1 && p.KW == 1) {
    if (av) return launch_splitk<og::kBGather, true, false, 1, 1>(variant, p, s);
    return launch_splitk<og::kBGather, false, false, 1, 1>(variant, p, s);
  }
  if (av) return launch_splitk<og::kBGather, true, false, 0, 0>(variant, p, s);
  return launch_splitk<og::kBGather, false, false, 0, 0>(variant, p, s);
}
#elif OG_UNIT == 14
void launch_halo_conv(int variant, int mode, const og::Problem &p, const HaloPlan &h, hipStream_t s) {
  if (halo_shape(variant).dpp) return launch_halo_dpp(variant, mode, p, h, s);
  if (mode == OG_MODE_EXACT) return launch_halo_exact(variant, p, h, s);
  if (variant == 26) return launch_halo_r<og::kFast, 1, 4, false>(p, h, s);
  if (variant == 27) return launch_halo_r<og::kFast, 2, 4, false>(p, h, s);
  return launch_halo_r<og::kFast, 1, 8, false>(p, h, s);
}
#elif OG_UNIT == 16
void launch_halo_exact(int variant, const og::Problem &p, const HaloPlan &h, hipStream_t s) {
  if (variant == 26) return launch_halo_r<og::kExact, 1, 4, false>(p, h, s);
  if (variant == 27) return launch_halo_r<og::kExact, 2, 4, false>(p, h, s);
  return launch_halo_r<og::kExact, 1, 8, false>(p, h, s);
}
#elif OG_UNIT == 17
template <int MODE>
static void launch_halo_dpp_mode(int variant, const og::Problem &p, const HaloPlan &h, hipStream_t s) {
  if (variant == 31) return launch_halo_r<MODE, 1, 4, true>(p, h, s);
  if (variant == 32) return launch_halo_r<MODE, 1, 8, true>(p, h, s);
  return launch_halo_r<MODE, 2, 4, true>(p, h, s);
}
void launch_halo_dpp(int variant, int mode, const og::Problem &p, const HaloPlan &h, hipStream_t s) {
  if (mode == OG_MODE_EXACT) return launch_halo_dpp_mode<og::kExact>(variant, p, h, s);
  launch_halo_dpp_mode<og::kFast>(variant, p, h, s);
}
#elif OG_UNIT == 15
template <int R>
static void launch_panel_r(int kind, bool bv, bool av, const og::Problem &p, hipStream_t s) {
  if (kind == og::kBMatrix) {
    if (bv && av) return launch_panel_shape<og::kBMatrix, R, true, true>(p, s);
    if (bv) return launch_panel_shape<og::kBMatrix, R, true, false>(p, s);
    if (av) return launch_panel_shape<og::kBMatrix, R, false, true>(p, s);
    return launch_panel_shape<og::kBMatrix, R, false, false>(p, s);
  }
  if (kind == og::kBPlanes) {
    if (bv && av) return launch_panel_shape<og::kBPlanes, R, true, true>(p, s);
    if (bv) return launch_panel_shape<og::kBPlanes, R, true, false>(p, s);
    if (av) return launch_panel_shape<og::kBPlanes, R, false, true>(p, s);
    return launch_panel_shape<og::kBPlanes, R, false, false>(p, s);
  }
  if (av) return launch_panel_shape<og::kBGather, R, false, true>(p, s);
  return launch_panel_shape<og::kBGather, R, false, false>(p, s);
}
void launch_panel(int variant, int kind, bool bv, bool av, const og::Problem &p, hipStream_t s) {
  if (variant == 29) return launch_panel_r<1>(kind, bv, av, p, s);
  return launch_panel_r<2>(kind, bv, av, p, s);
}
#else
#error "unknown OG_UNIT"
#endif

}  // namespace og::host
