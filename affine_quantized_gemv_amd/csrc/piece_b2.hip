// Instantiation of the 16-byte-piece streaming kernels for affine 2-bit codes.
#include "piece_kernel.h"

namespace aqg {
template <>
hipError_t launch_piece<2, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_piece_impl<2, false>(a, c, s);
}
}  // namespace aqg
