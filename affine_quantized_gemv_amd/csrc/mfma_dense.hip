// Instantiation of the matrix-core kernels for the dense bf16 GEMV and the
// fused SwiGLU (M padded to 16 or 32).
#include "mfma_kernel.h"

namespace aqg {
template <>
hipError_t launch_mfma<false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_impl<false>(a, c, s);
}
template <>
hipError_t launch_mfma<true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_impl<true>(a, c, s);
}
}  // namespace aqg
