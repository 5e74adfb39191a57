// Instantiation of the fused SwiGLU over affine gate and up matrices of 3,
// 5, 6 and 7 bits on the small-N affine matrix-core kernel.
#include "affine_split.h"

namespace aqg {
#define AQG_SPLIT_ODD_SW(B)                                                                   \
    template <>                                                                               \
    hipError_t launch_affine_split<B, true>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s) \
    {                                                                                         \
        return detail::launch_affine_split_impl<B, 2>(a, c, s);                               \
    }
AQG_SPLIT_ODD_SW(3)
AQG_SPLIT_ODD_SW(5)
AQG_SPLIT_ODD_SW(6)
AQG_SPLIT_ODD_SW(7)
#undef AQG_SPLIT_ODD_SW
}  // namespace aqg
