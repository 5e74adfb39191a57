// Instantiation of the persistent matrix-core streaming kernels and the
// small-N k-split matrix-core kernels (dense bf16 GEMV and fused SwiGLU, M
// padded to 16 or 32).
#include "mfma_split.h"

namespace aqg {
template <>
hipError_t launch_mfma_stream<false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_stream_impl<false>(a, c, s);
}
template <>
hipError_t launch_mfma_stream<true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_stream_impl<true>(a, c, s);
}
template <>
hipError_t launch_mfma_split<false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_split_impl<false>(a, c, s);
}
template <>
hipError_t launch_mfma_split<true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_split_impl<true>(a, c, s);
}
}  // namespace aqg
