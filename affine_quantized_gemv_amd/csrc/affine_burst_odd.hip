// Instantiation of the multi-tile affine matrix-core kernels for 3-, 5-, 6-
// and 7-bit codes.
#include "affine_burst.h"

namespace aqg {
template <int BITS>
hipError_t launch_affine_burst(const ProjArgs& a, const LaunchCfg&, hipStream_t s)
{
    return detail::launch_affine_burst_impl<BITS>(a, s);
}
template hipError_t launch_affine_burst<3>(const ProjArgs&, const LaunchCfg&, hipStream_t);
template hipError_t launch_affine_burst<5>(const ProjArgs&, const LaunchCfg&, hipStream_t);
template hipError_t launch_affine_burst<6>(const ProjArgs&, const LaunchCfg&, hipStream_t);
template hipError_t launch_affine_burst<7>(const ProjArgs&, const LaunchCfg&, hipStream_t);
}  // namespace aqg
