// Instantiation of the projection kernels for affine 3-bit codes.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<3, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<3, false>(a, c, s);
}
template <>
hipError_t launch_stream<3, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<3, false>(a, c, s);
}
}  // namespace aqg
