// Instantiation of the projection kernels for affine 2-bit codes.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<2, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<2, false>(a, c, s);
}
template <>
hipError_t launch_stream<2, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<2, false>(a, c, s);
}
}  // namespace aqg
