// Matrix-core path for M = 9..32 (M padded to 16 or 32): dense bf16 GEMV and
// fused SwiGLU on gfx950 with v_mfma_f32_16x16x32_bf16.
//
// With 16 or 32 activation rows the projection is a real (skinny) dense
// contraction: y^T[N, M] = W[N, K] . x^T[K, M].  One MFMA multiplies a 16-row
// by 32-k tile of W (the A operand, streamed from HBM, 16 bytes per lane) by
// a 32-k by 16-column tile of x^T (the B operand, read from LDS) into a
// 16 x 16 fp32 accumulator.  Operand layouts (CDNA4 16x16x32 bf16):
//   A: lane l holds row (l % 16), k = 8*(l/16) .. 8*(l/16)+7,
//   B: lane l holds column (l % 16), the same 8 k,
//   D: lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
//
// Workgroup = NR row groups x NK k-splits wavefronts.  Each row group owns
// 16*RT rows.  x (all M rows, one K-tile) is staged once per workgroup in
// fragment order: for k-step s (32 k) and column block mb, the 64 lanes'
// 16-byte B operands are contiguous.  A wavefront walks the K-tile's k-steps
// wk, wk+NK, ... keeping D k-steps of weights in flight; when NK > 1 the
// partial accumulators of the k-splits are summed through LDS in a fixed
// order (split 0 + split 1 + ...), so results are deterministic.
//
// Shapes and fused up/gate SwiGLU: AstrAI decode_linear_benchmark.md (commit
// message; M = 1..32 decode shapes).  Weights are read exactly once; x and the
// accumulators never leave the chip.
#pragma once
#include "aqg_device.h"
#include "kernels.h"

namespace aqg {
namespace detail {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaMaxThreads = 512;

__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int MT, int RT, bool SWIGLU>
__global__ void __launch_bounds__(kMfmaMaxThreads) mfma_dense_kernel(ProjArgs a)
{
    extern __shared__ u32x4_t lds_v4[];
    constexpr int MB = MT / 16;          // 16-column blocks of x^T
    constexpr int S = SWIGLU ? 2 : 1;    // weight streams
    constexpr int D = 4;                 // k-steps of weights in flight per wavefront

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nk_log2 = a.ksplit_log2;   // k-splits per row group
    const int NK = 1 << nk_log2;
    const int NR = (blockDim.x >> 6) >> nk_log2;
    const int wr = wave >> nk_log2;
    const int wk = wave & (NK - 1);
    const int q = lane >> 4;             // k sub-block (A, B) / row quad (D)
    const int c16 = lane & 15;           // A row / B and D column

    const int64_t tile0 = ((int64_t)blockIdx.x * NR + wr) * (16 * RT);
    const uint16_t* wrow[S][RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        int64_t n = tile0 + 16 * r + c16;
        if (n >= a.N) n = a.N - 1;       // clamp: load, never store
        wrow[0][r] = reinterpret_cast<const uint16_t*>(a.w0) + n * a.K + 8 * q;
        if constexpr (SWIGLU) wrow[1][r] = reinterpret_cast<const uint16_t*>(a.w1) + n * a.K + 8 * q;
    }

    f32x4_t acc[S][RT][MB];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[s][r][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wb[D][S][RT];

    for (int kt = 0; kt < a.K; kt += a.KT) {
        const int kw = min(a.KT, a.K - kt);
        const int ks = kw >> 5;                        // k-steps in this tile
        const int nsteps = (ks - wk + NK - 1) >> nk_log2;  // this wavefront's k-steps

        auto fetch = [&](int d, int j) __attribute__((always_inline)) {
            const int koff = kt + 32 * j;
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    wb[d][s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wrow[s][r] + koff));
        };

        // Stage x: task (m, c8) -> 8 k of row m; zero rows m >= M.  Each
        // thread loads XB tasks at once (one latency, not XB), the first batch
        // before the first weight loads are issued.
        constexpr int XB = 8;
        const int c8n = kw >> 3;
        const int ntask = MT * c8n;
        const int nthr = blockDim.x;
        u32x4_t xr[XB];
        auto xload = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * nthr;
                xr[i] = u32x4_t{0u, 0u, 0u, 0u};
                if (t < ntask) {
                    const int m = t / c8n, c8 = t - m * c8n;
                    if (m < a.M) xr[i] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)m * a.K + kt + 8 * c8);
                }
            }
        };
        auto xstore = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * nthr;
                if (t < ntask) {
                    const int m = t / c8n, c8 = t - m * c8n;
                    const int s = c8 >> 2, qq = c8 & 3;
                    lds_v4[(s * MB + (m >> 4)) * 64 + qq * 16 + (m & 15)] = xr[i];
                }
            }
        };
        xload(threadIdx.x);
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int d = decltype(Dd)::value;
            if (d < nsteps) fetch(d, wk + d * NK);
        });
        if (kt > 0) __syncthreads();
        xstore(threadIdx.x);
        for (int t0 = threadIdx.x + XB * nthr; t0 < ntask; t0 += XB * nthr) {
            xload(t0);
            xstore(t0);
        }
        __syncthreads();

        for (int base = 0; base < nsteps; base += D) {
            static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
                constexpr int d = decltype(Dd)::value;
                const int i = base + d;
                if (i < nsteps) {
                    const int j = wk + i * NK;
                    u32x4_t bfrag[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) bfrag[mb] = lds_v4[(j * MB + mb) * 64 + lane];
#pragma unroll
                    for (int s = 0; s < S; ++s)
#pragma unroll
                        for (int r = 0; r < RT; ++r)
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb)
                                acc[s][r][mb] = mfma16x16x32(wb[d][s][r], bfrag[mb], acc[s][r][mb]);
                    if (i + D < nsteps) fetch(d, j + D * NK);
                }
            });
        }
    }

    // Sum the k-splits of each row group in a fixed order through LDS.
    if (NK > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds_v4);
        constexpr int PER = S * RT * MB * 4;               // floats per lane
        float* mine = red + ((size_t)(wr * NK + wk) * PER) * 64;
        if (wk != 0) {
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            mine[(((s * RT + r) * MB + mb) * 4 + i) * 64 + lane] = acc[s][r][mb][i];
        }
        __syncthreads();
        if (wk != 0) return;
        for (int w = 1; w < NK; ++w) {
            const float* other = red + ((size_t)(wr * NK + w) * PER) * 64;
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[s][r][mb][i] += other[(((s * RT + r) * MB + mb) * 4 + i) * 64 + lane];
        }
    }

    // Epilogue: lane holds rows tile0 + 16r + 4q + i, column m = 16 mb + c16.
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = 16 * mb + c16;
            if (m >= a.M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = tile0 + 16 * r + 4 * q + i;
                if (n >= a.N) continue;
                float v = acc[0][r][mb][i];
                if constexpr (SWIGLU) {
                    const float g = v;
                    v = (g / (1.0f + __expf(-g))) * acc[1][r][mb][i];
                }
                const size_t o = (size_t)m * a.N + n;
                if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = v;
                else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(v);
            }
        }
}

template <int MT, int RT, bool SW>
hipError_t launch_mfma_one(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    hipLaunchKernelGGL((mfma_dense_kernel<MT, RT, SW>), dim3(c.blocks), dim3(64 * c.nwaves), c.lds, s, a);
    return hipGetLastError();
}

template <bool SW>
hipError_t launch_mfma_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (c.MT == 16) return c.R == 2 ? launch_mfma_one<16, 2, SW>(a, c, s) : launch_mfma_one<16, 1, SW>(a, c, s);
    if (c.MT == 32) return c.R == 2 ? launch_mfma_one<32, 2, SW>(a, c, s) : launch_mfma_one<32, 1, SW>(a, c, s);
    return hipErrorInvalidValue;
}

}  // namespace detail
}  // namespace aqg
