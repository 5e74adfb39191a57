// Instantiation of the 16-byte-piece streaming kernels for the fused SwiGLU
// over affine 4-bit gate and up matrices.
#include "piece_kernel.h"

namespace aqg {
template <>
hipError_t launch_piece<4, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_piece_impl<4, true>(a, c, s);
}
}  // namespace aqg
