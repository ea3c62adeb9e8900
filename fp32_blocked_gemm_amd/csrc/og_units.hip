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
#else
#error "unknown OG_UNIT"
#endif

}  // namespace og::host
