// Instantiation of the small-N affine matrix-core kernels (k split over one
// workgroup per 16-row tile) for 3-, 5-, 6- and 7-bit codes.
#include "affine_split.h"

namespace aqg {
#define AQG_SPLIT_ODD(B)                                                                       \
    template <>                                                                                \
    hipError_t launch_affine_split<B, false>(const ProjArgs& a, const LaunchCfg& c, hipStream_t s) \
    {                                                                                          \
        return detail::launch_affine_split_impl<B, 1>(a, c, s);                                \
    }
AQG_SPLIT_ODD(3)
AQG_SPLIT_ODD(5)
AQG_SPLIT_ODD(6)
AQG_SPLIT_ODD(7)
#undef AQG_SPLIT_ODD
}  // namespace aqg
