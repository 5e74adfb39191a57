// Instantiation of the affine prompt GEMM (pre-pass and main kernel) for
// 4-bit codes.
#include "affine_gemm.h"

namespace aqg {
template <>
hipError_t launch_affine_gemm<4>(const GemmArgs& a, hipStream_t s)
{
    return detail::launch_affine_gemm_impl<4>(a, s);
}
}  // namespace aqg
