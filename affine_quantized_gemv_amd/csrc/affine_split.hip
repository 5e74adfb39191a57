// Instantiation of the small-N affine matrix-core kernels (k split over one
// workgroup per 16-row tile) for 2-, 4- and 8-bit codes.
#include "affine_split.h"

namespace aqg {
template <>
hipError_t launch_affine_split<2, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<2, 1>(a, c, s);
}
template <>
hipError_t launch_affine_split<4, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<4, 1>(a, c, s);
}
template <>
hipError_t launch_affine_split<8, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<8, 1>(a, c, s);
}
}  // namespace aqg
