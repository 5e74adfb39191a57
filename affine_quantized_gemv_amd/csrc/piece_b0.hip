// Instantiation of the 16-byte-piece streaming kernels for dense bf16 weights.
#include "piece_kernel.h"

namespace aqg {
template <>
hipError_t launch_piece<0, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_piece_impl<0, false>(a, c, s);
}
}  // namespace aqg
