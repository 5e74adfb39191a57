// Instantiation of the dense matrix-core tile kernels (M padded to 16 or 32;
// K = 512, 1024, 1536, 2048).
#include "mfma_tile.h"

namespace aqg {
hipError_t launch_mfma_tile(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    return detail::launch_mfma_tile_impl(a, c, s);
}
}  // namespace aqg
