// Instantiation of the affine matrix-core tile kernels for 3-bit codes (M
// padded to 16 or 32).
#include "affine_tile.h"

namespace aqg {
template <>
hipError_t launch_affine_tile<3>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_tile_impl<3>(a, c, s);
}
}  // namespace aqg
