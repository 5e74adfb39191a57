// Instantiation of the projection kernels for the fused SwiGLU over affine
// 5-bit gate and up matrices.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<5, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<5, true>(a, c, s);
}
template <>
hipError_t launch_stream<5, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<5, true>(a, c, s);
}
}  // namespace aqg
