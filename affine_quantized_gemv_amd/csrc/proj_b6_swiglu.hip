// Instantiation of the projection kernels for the fused SwiGLU over affine
// 6-bit gate and up matrices.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<6, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<6, true>(a, c, s);
}
template <>
hipError_t launch_stream<6, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<6, true>(a, c, s);
}
}  // namespace aqg
