// Device-side helpers for the gfx950 (CDNA4) projection kernels: bit windows
// over packed code streams, bf16x2 dot products, bf16 conversions and
// wavefront-segment reductions with DPP.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their
// maximum, i.e. not waited for): gfx9-family encoding.
constexpr int kWaitVmcnt0 = 0x0F70;

// (a & m) | c -- one v_and_or_b32.  Written as asm because, with m and c
// compile-time constants, the compiler would otherwise emit v_and_b32 +
// v_or_b32 with literal operands (a 3-operand VALU op cannot take literals
// here); m goes to a scalar register and c to a vector register, both loop
// invariant.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

// 32 consecutive bits of a group's LSB-first code stream (NW words), starting
// at stream bit ST; bits outside the stream read as zero.  ST is a compile-time
// constant, so this is one v_alignbit_b32, one shift, or a plain register.
template <int ST, int NW>
__device__ __forceinline__ uint32_t win(const uint32_t* w)
{
    static_assert(ST > -32 && ST < 32 * NW, "window outside the group");
    if constexpr (ST < 0) {
        return w[0] << (-ST);
    } else if constexpr (ST % 32 == 0) {
        return w[ST / 32];
    } else if constexpr ((ST >> 5) + 1 < NW) {
        return __builtin_amdgcn_alignbit(w[(ST >> 5) + 1], w[ST >> 5], ST & 31);
    } else {
        return w[ST >> 5] >> (ST & 31);
    }
}

// c + a.lo*b.lo + a.hi*b.hi with bf16 halves, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The bf16 pair a zero code field places: (128, 128).
constexpr uint32_t kZeroCodePair = 0x43004300u;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even; NaN becomes a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Exact scaling of a bf16 by 2^E (E a small compile-time integer) returning a
// bf16 bit pattern.  Exact for normal inputs whose result stays normal.
template <int E>
__device__ __forceinline__ uint32_t bf16_scale_pow2(uint32_t h)
{
    if constexpr (E == 0) {
        return h & 0xFFFFu;
    } else {
        constexpr float s = E > 0 ? (float)(1u << (E > 0 ? E : 0)) : 1.0f / (float)(1u << (E < 0 ? -E : 0));
        return __float_as_uint(bf16_to_f32(h & 0xFFFFu) * s) >> 16;
    }
}

// (bound_ctrl set: a source lane that is out of its row or inactive reads 0.
// The patterns used here never leave the row, and with it set the compiler
// folds the move into the add that consumes it, one instruction per step.)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned segments of 2^L lanes (L <= 4), result in every lane of the
// segment.  The tree is the same for every value and every lane: pairs of
// lanes, then quads, then the two quads of a half-row (row_half_mirror), then
// the two halves of a 16-lane row (row_mirror).  Each step adds two equal
// partial sums in either order, so all lanes end with bit-identical totals.
__device__ __forceinline__ float segment_sum(float v, int L)
{
    if (L >= 1) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    if (L >= 2) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    if (L >= 3) v += dpp_f32<0x141>(v);  // row_half_mirror
    if (L >= 4) v += dpp_f32<0x140>(v);  // row_mirror
    return v;
}

// Keep the code on each side of this point on its own side: a compiler
// memory barrier (no load moves across it) plus a machine-scheduler barrier.
// Used between the chunks of an unrolled unit so that each chunk's operands
// and LDS reads stay short-lived.
__device__ __forceinline__ void code_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Make v's current value an input and output of an empty asm statement: every
// instruction that produces v is placed before this point and every use after.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int I> struct Int { static constexpr int value = I; };
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(Int<B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace aqg
