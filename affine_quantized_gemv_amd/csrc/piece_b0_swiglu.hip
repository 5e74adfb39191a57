// Instantiation of the 16-byte-piece streaming kernels for the fused SwiGLU (dense bf16 gate and up weights).
#include "piece_kernel.h"

namespace aqg {
template <>
hipError_t launch_piece<0, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_piece_impl<0, true>(a, c, s);
}
}  // namespace aqg
