// Instantiation of the multi-tile affine matrix-core kernels for 2-, 4- and
// 8-bit codes.
#include "affine_burst.h"

namespace aqg {
template <int BITS>
hipError_t launch_affine_burst(const ProjArgs& a, const LaunchCfg&, hipStream_t s)
{
    return detail::launch_affine_burst_impl<BITS>(a, s);
}
template hipError_t launch_affine_burst<2>(const ProjArgs&, const LaunchCfg&, hipStream_t);
template hipError_t launch_affine_burst<4>(const ProjArgs&, const LaunchCfg&, hipStream_t);
template hipError_t launch_affine_burst<8>(const ProjArgs&, const LaunchCfg&, hipStream_t);
}  // namespace aqg
