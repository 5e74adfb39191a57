// Instantiation of the projection kernels for affine 8-bit codes.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<8, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<8, false>(a, c, s);
}
template <>
hipError_t launch_stream<8, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<8, false>(a, c, s);
}
}  // namespace aqg
