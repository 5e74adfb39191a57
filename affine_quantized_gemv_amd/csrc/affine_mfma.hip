// Instantiation of the affine matrix-core kernels for 4-bit codes (M padded
// to 16 or 32; every chunk-table size).
#include "affine_mfma.h"

namespace aqg {
template <>
hipError_t launch_affine_mfma<4>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_mfma_impl<4>(a, c, s);
}
}  // namespace aqg
