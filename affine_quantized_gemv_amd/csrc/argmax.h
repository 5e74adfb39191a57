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

// Combine with the lane a DPP pattern pairs it with (all lanes active; the
// patterns used stay within a 16-lane row).
template <int CTRL>
__device__ __forceinline__ void amx_dpp(float& bv, int& bi)
{
    const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, true));
    const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, true);
    amx_take(bv, bi, ov, oi);
}

// Every lane of each 16-lane row ends with the row's best: pairs, quads, the
// two quads of a half-row, the two halves (the segment-sum tree of the
// GEMVs, with the total order's combine in place of the add).
__device__ __forceinline__ void amx_row(float& bv, int& bi)
{
    amx_dpp<0xB1>(bv, bi);    // quad_perm [1,0,3,2]
    amx_dpp<0x4E>(bv, bi);    // quad_perm [2,3,0,1]
    amx_dpp<0x141>(bv, bi);   // row_half_mirror
    amx_dpp<0x140>(bv, bi);   // row_mirror
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
