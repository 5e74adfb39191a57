// Instantiation of the 4-bit affine matrix-core kernels (M padded to 16 or 32).
#include "affine_mfma.h"

namespace aqg {
hipError_t launch_affine4_mfma(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_affine_mfma_impl(a, c, s);
}
}  // namespace aqg
