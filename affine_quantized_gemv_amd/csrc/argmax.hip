// Reductions of row-argmax partials (argmax.h): the final combine over the
// producers of a fused GEMV epilogue, and the per-chunk maxima of an fp32
// output for kernels without a fused epilogue.
#include "argmax.h"
#include "kernels.h"

namespace aqg {
namespace detail {
namespace {

// The order (value, then lower index) is total, so these combines give the
// same answer in any grouping; they are written for latency: every thread
// issues kArgmaxUnroll independent loads before combining them (a loop of
// one dependent load per step took 4.5 us over 2048 partials and 10 us over
// 7168), and the combines run on DPP lane moves where they stay in a row.
constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxUnroll = 8;

// Block-wide combine of one (value, index) per thread; thread 0 returns it.
// Within a wavefront: the row tree, then lane swaps across 16 and 32; across
// the wavefronts: wavefront 0 takes their results one per lane and runs the
// row tree again (a serial loop over them took ~1 us of dependent LDS reads).
__device__ __forceinline__ void amx_block(float& bv, int& bi)
{
    constexpr int NWV = kArgmaxThreads / 64;
    static_assert(NWV <= 16, "one wavefront result per lane of a row");
    __shared__ float sv[NWV];
    __shared__ int si[NWV];
    amx_row(bv, bi);
    amx_xor(bv, bi, 16);
    amx_xor(bv, bi, 32);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (wave == 0) {
        bv = lane < NWV ? sv[lane] : amx_neutral_value();
        bi = lane < NWV ? si[lane] : kAmxNoIndex;
        amx_row(bv, bi);
    }
}

// One workgroup per row m: the best of the P producers' partials.
__global__ void __launch_bounds__(kArgmaxThreads) argmax_final_kernel(const int2* __restrict__ part, int64_t slots,
                                                                      int64_t P, float* __restrict__ val,
                                                                      int* __restrict__ idx)
{
    const int m = blockIdx.x;
    const int2* row = part + m * slots;
    float bv = amx_neutral_value();
    int bi = kAmxNoIndex;
    for (int64_t p0 = threadIdx.x; p0 < P; p0 += (int64_t)kArgmaxThreads * kArgmaxUnroll) {
        int2 e[kArgmaxUnroll];
#pragma unroll
        for (int u = 0; u < kArgmaxUnroll; ++u) {
            const int64_t p = p0 + (int64_t)u * kArgmaxThreads;
            e[u] = p < P ? row[p] : make_int2(__float_as_int(amx_neutral_value()), kAmxNoIndex);
        }
#pragma unroll
        for (int u = 0; u < kArgmaxUnroll; ++u) amx_take(bv, bi, __int_as_float(e[u].x), e[u].y);
    }
    amx_block(bv, bi);
    if (threadIdx.x == 0) {
        val[m] = bv;
        idx[m] = bi;
    }
}

// Workgroup (c, m): the best of y[m][c*chunk .. (c+1)*chunk) as producer c.
__global__ void __launch_bounds__(kArgmaxThreads) argmax_rows_kernel(const float* __restrict__ y, int N, int chunk,
                                                                     int2* __restrict__ part, int64_t slots)
{
    const int c = blockIdx.x, m = blockIdx.y;
    const int64_t n0 = (int64_t)c * chunk;
    const int64_t n1 = n0 + chunk < N ? n0 + chunk : N;
    const float* yr = y + (int64_t)m * N;
    float bv = amx_neutral_value();
    int bi = kAmxNoIndex;
    for (int64_t q0 = n0 + threadIdx.x; q0 < n1; q0 += (int64_t)kArgmaxThreads * kArgmaxUnroll) {
        float v[kArgmaxUnroll];
#pragma unroll
        for (int u = 0; u < kArgmaxUnroll; ++u) {
            const int64_t n = q0 + (int64_t)u * kArgmaxThreads;
            v[u] = n < n1 ? yr[n] : amx_neutral_value();
        }
#pragma unroll
        for (int u = 0; u < kArgmaxUnroll; ++u) {
            const int64_t n = q0 + (int64_t)u * kArgmaxThreads;
            amx_take(bv, bi, v[u], n < n1 ? (int)n : kAmxNoIndex);
        }
    }
    amx_block(bv, bi);
    if (threadIdx.x == 0) part[m * slots + c] = make_int2(__float_as_int(bv), bi);
}

}  // namespace
}  // namespace detail

hipError_t launch_argmax_final(const void* part, int64_t slots, int64_t P, int M, float* val, int* idx,
                               hipStream_t s)
{
    if (P < 1 || P > slots) return hipErrorInvalidValue;
    hipLaunchKernelGGL(detail::argmax_final_kernel, dim3(M), dim3(detail::kArgmaxThreads), 0, s,
                       static_cast<const int2*>(part), slots, P, val, idx);
    return hipGetLastError();
}

hipError_t launch_argmax_rows(const float* y, int M, int N, int chunk, void* part, int64_t slots, hipStream_t s)
{
    const int chunks = (N + chunk - 1) / chunk;
    if (chunks > slots) return hipErrorInvalidValue;
    hipLaunchKernelGGL(detail::argmax_rows_kernel, dim3(chunks, M), dim3(detail::kArgmaxThreads), 0, s, y, N, chunk,
                       static_cast<int2*>(part), slots);
    return hipGetLastError();
}

}  // namespace aqg
