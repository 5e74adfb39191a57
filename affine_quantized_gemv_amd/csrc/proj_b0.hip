// Instantiation of the projection kernels for dense bf16.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<0, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<0, false>(a, c, s);
}
template <>
hipError_t launch_stream<0, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<0, false>(a, c, s);
}
}  // namespace aqg
