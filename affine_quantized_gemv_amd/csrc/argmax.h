// Device helpers for the row argmax fused into the GEMV epilogues: a running
// (value, index) maximum in which the lower index wins on equal values
// (nvfp4-megamoe-kernel commit log, "Router: full kernel stack", Step 2:
// topk_select keeps the lower index on ties).  The order is total on
// (value, -index) for non-NaN values, so the result does not depend on the
// order in which partial maxima are combined.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqg {
namespace detail {

constexpr int kArgmaxRows = 32;        // partial entries per producer (M <= 32)

__device__ __forceinline__ void amx_take(float& bv, int& bi, float v, int i)
{
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// Combine with the lane `mask` away (xor), e.g. a butterfly over lanes.
__device__ __forceinline__ void amx_xor(float& bv, int& bi, int mask)
{
    const float ov = __shfl_xor(bv, mask);
    const int oi = __shfl_xor(bi, mask);
    amx_take(bv, bi, ov, oi);
}

// Partials are laid out row-major, [m][slots]: the final reduction of a row
// reads one contiguous run.
__device__ __forceinline__ void amx_store(void* amx, int64_t slots, int64_t producer, int m, float v, int i)
{
    reinterpret_cast<int2*>(amx)[m * slots + producer] = make_int2(__float_as_int(v), i);
}

__device__ __forceinline__ float amx_neutral_value() { return -__builtin_huge_valf(); }
constexpr int kAmxNoIndex = 0x7FFFFFFF;

}  // namespace detail
}  // namespace aqg
