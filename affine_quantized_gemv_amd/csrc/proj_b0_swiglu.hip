// Instantiation of the projection kernels for dense bf16 SwiGLU.
#include "stream_kernel.h"

namespace aqg {
template <>
hipError_t launch_bits<0, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_bits_impl<0, true>(a, c, s);
}
template <>
hipError_t launch_stream<0, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_stream_impl<0, true>(a, c, s);
}
}  // namespace aqg
