// Instantiation of the small-N affine matrix-core kernels for the fused
// SwiGLU over affine 2-, 4- and 8-bit gate and up matrices.
#include "affine_split.h"

namespace aqg {
template <>
hipError_t launch_affine_split<2, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<2, 2>(a, c, s);
}
template <>
hipError_t launch_affine_split<4, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<4, 2>(a, c, s);
}
template <>
hipError_t launch_affine_split<8, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_split_impl<8, 2>(a, c, s);
}
}  // namespace aqg
