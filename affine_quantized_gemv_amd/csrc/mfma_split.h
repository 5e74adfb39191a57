// Matrix-core kernel for small-N dense projections and fused SwiGLU at
// M = 9..32 (from M = 3 on wide matrices, from M = 5 on short ones; M padded
// to 16 or 32) on gfx950:
// one workgroup per 16-row tile, K split over NKS wavefronts.
//
// A small matrix (a few MB) is latency-bound: what matters is how soon every
// CU has its loads in flight.  Here nothing waits before the loads: each
// wavefront issues, at once, the A operands of its SPW k-steps (whole-line
// pair loads with the DPP half-swap, as in mfma_stream.h) and the x^T B
// operands of the same k-steps straight from global memory (L2-resident; no
// LDS staging, no barrier), then runs its MFMAs.  The NKS partial 16 x MT
// tiles are summed through LDS in a fixed order (wavefront 0 + 1 + ...), so
// results are deterministic and the same for every M of the path.
//
// Shapes and fused up/gate SwiGLU: AstrAI decode_linear_benchmark.md (commit
// message; q/k/v/out, MLP shapes at M = 1..32).
#pragma once
#include "mfma_stream.h"

namespace aqg {
namespace detail {

constexpr int kMfmaSplitMaxWaves = 16;

// CW > 0 (the 16-column kernel serving up to 2 CW columns): workgroup b
// takes column block (b / 8) % 2, columns [CW, 2 CW) for block 1, of row tile
// 8 (b / 16) + b % 8, so the two column blocks of a tile run on one XCD
// (workgroup b runs on XCD b % 8) and the second read of the tile's weights
// finds them in that XCD's L2.  Twice the workgroups, each with half of the
// x^T traffic.  An output's MFMA chain does not depend on its column, so
// results are those of the unsplit kernel.
// SEG: a multi-projection launch (the tile's projection looked up in the
// table at entry); a separate instantiation, so single projections load no
// table before their first weight loads.
template <int MT, bool SWIGLU, int SPW, int CW = 0, bool SEG = false>
__global__ void __launch_bounds__(64 * kMfmaSplitMaxWaves) mfma_split_kernel(ProjArgs a)
{
    extern __shared__ float lds_red[];
    int64_t tile = blockIdx.x;
    if constexpr (CW > 0) {
        static_assert(MT == 16 && CW <= 16, "column blocks of a 16-column kernel");
        tile = (int64_t)(blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
        if (tile * 16 >= a.N) return;            // whole workgroup, before any barrier
    }
    // this tile's matrix, scales, biases, output and row count: those of its
    // projection in a multi-projection launch (locals: the kernel never
    // writes its argument block)
    SegView sv{a.w0, a.scales, a.biases, a.y, a.N, tile * 16};
    if constexpr (SEG) sv = seg_view(a, tile * 16);
    const int64_t n0 = sv.n0;
    const int N_ = sv.N;
    const void* const w0_ = sv.w;
    const uint16_t* x_ = a.x;
    void* y_ = sv.y;
    int M_ = a.M;
    if constexpr (CW > 0) {
        if ((blockIdx.x >> 3) & 1) {
            x_ += (size_t)CW * a.K;
            y_ = static_cast<char*>(y_) + (size_t)CW * N_ * (a.out_f32 ? 4 : 2);
            M_ -= CW;
        } else if (M_ > CW) {
            M_ = CW;
        }
    }
    constexpr int NB = MT / 16;
    constexpr int S = SWIGLU ? 2 : 1;
    constexpr int NP = SPW / 2;                  // k-step pairs per wavefront
    static_assert(SPW % 2 == 0, "k-steps come in pairs");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nks = blockDim.x >> 6;
    const int c = lane >> 4;
    const int r = lane & 15;
    const int h = lane & 15;
    const int64_t row_bytes = (int64_t)a.K * 2;
    const int s0 = wave * SPW;                   // first k-step of this wavefront

    // A: pair p covers k-steps s0 + 2p, s0 + 2p + 1 (64 k, 128 bytes per row)
    const uint32_t voff = (uint32_t)((h & 7) * row_bytes + 16 * ((h < 8 ? 0 : 4) + c));
    // rows 8..15: the row offset goes in the vector offset, which is the
    // part of the address the buffer range check covers
    const uint32_t voff_hi = voff + (uint32_t)(8 * row_bytes);
    u32x4_t wa[NP][S][2];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const __amdgpu_buffer_rsrc_t rs =
            tile_rsrc(static_cast<const char*>(s == 0 ? w0_ : a.w1) + n0 * row_bytes, (N_ - n0) * row_bytes);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int koff = 64 * (s0 + 2 * p);  // bytes: 32 k per step, 2 bytes each
            wa[p][s][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, koff, kLoadNT));
            wa[p][s][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff_hi, koff, kLoadNT));
        }
    }
    // B: lane (c, column r) of block b holds x[16b + r][32 s + 8c .. + 7]
    u32x4_t xb[SPW][NB];
#pragma unroll
    for (int t = 0; t < SPW; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int m = 16 * b + r;
            xb[t][b] = u32x4_t{0u, 0u, 0u, 0u};
            if (m < M_)
                xb[t][b] = *reinterpret_cast<const u32x4_t*>(x_ + (size_t)m * a.K + 32 * (s0 + t) + 8 * c);
        }

    const bool hi8 = (lane & 8) != 0;
    f32x4_t acc[S][NB];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            u32x4_t A0, A1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t l0 = wa[p][s][0][i], l1 = wa[p][s][1][i];
                const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0, 0x128, 0xF, 0xF, false);
                const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1, 0x128, 0xF, 0xF, false);
                A0[i] = hi8 ? r1 : l0;
                A1[i] = hi8 ? l1 : r0;
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                acc[s][b] = mfma16x16x32(A0, xb[2 * p][b], acc[s][b]);
                acc[s][b] = mfma16x16x32(A1, xb[2 * p + 1][b], acc[s][b]);
            }
        }

    // fixed-order sum of the k-splits: every wavefront stores its partial
    // tile (rows of 65 floats: conflict-free reads below), then every thread
    // adds one output's partials in order 0, 1, ..., nks-1 and stores it
    constexpr int PER = S * NB * 4;              // floats per lane
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_red[((size_t)(wave * PER) + (s * NB + b) * 4 + i) * 65 + lane] = acc[s][b][i];
    __syncthreads();
    // output (m, n0 + n16) lives in lane (n16 / 4) * 16 + m % 16, element
    // (block m / 16, n16 % 4) of each partial
    for (int o = threadIdx.x; o < 16 * MT; o += blockDim.x) {
        const int m = o >> 4, n16 = o & 15;
        const int j0 = ((m >> 4) * 4 + (n16 & 3)) * 65 + (n16 >> 2) * 16 + (m & 15);
        float v = lds_red[j0];
        float u = 0.f;
        if constexpr (SWIGLU) u = lds_red[j0 + NB * 4 * 65];
        for (int w = 1; w < nks; ++w) {
            v += lds_red[(size_t)(w * PER) * 65 + j0];
            if constexpr (SWIGLU) u += lds_red[(size_t)(w * PER + NB * 4) * 65 + j0];
        }
        const int64_t n = n0 + n16;
        if (m >= M_ || n >= N_) continue;
        if constexpr (SWIGLU) v = (v / (1.0f + __expf(-v))) * u;
        const size_t oi = (size_t)m * N_ + n;
        if (a.out_f32) reinterpret_cast<float*>(y_)[oi] = v;
        else reinterpret_cast<uint16_t*>(y_)[oi] = f32_to_bf16_rne(v);
    }
}

// k-steps per wavefront for a K: the smallest of 2, 4, 6, 8 that splits the
// K/32 steps over at most 16 wavefronts (0 if none does; SwiGLU stops at 6,
// where its two weight streams still fit in registers at M = 32).
inline int mfma_split_spw(int K, bool swiglu)
{
    if (K % 64 != 0) return 0;
    const int ks = K / 32;
    for (int spw : {2, 4, 6, 8})
        if (ks % spw == 0 && ks / spw <= kMfmaSplitMaxWaves) return (swiglu && spw > 6) ? 0 : spw;
    return 0;
}

template <int MT, bool SW, int SPW, bool SEG>
hipError_t launch_mfma_split_seg(const ProjArgs& a, hipStream_t s)
{
    const int nks = (a.K / 32) / SPW;
    const int64_t tiles = ((int64_t)a.N + 15) / 16;
    // With at most half as many row tiles as CUs, M = 17..32 runs the
    // 16-column kernel once per 16-column block and M = 9..16 once per
    // 8-column block (q/k/v/o 1536 x 1536 at M = 32: 6.7 -> 5.2 us; down
    // 1536 x 4096: 13.9 -> 9.9 us).  With more tiles the second read of the
    // weights costs more than it saves (up/gate 4096 x 1536 at M = 32: 7.2 ->
    // 8.0 us), so the columns stay in one workgroup.
    // M = 5..8 likewise once per 4-column block.
    if (MT == 32 || a.M > 4) {
        int cus = 0;
        hipError_t e = device_cus(cus);
        if (e != hipSuccess) return e;
        if (2 * tiles <= cus) {
            const size_t lds = (size_t)nks * (SW ? 2 : 1) * 4 * 65 * 4;
            const int64_t blocks = (tiles + 7) / 8 * 16;
            if constexpr (MT == 32)
                hipLaunchKernelGGL((mfma_split_kernel<16, SW, SPW, 16, SEG>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
            else if (a.M > 8)
                hipLaunchKernelGGL((mfma_split_kernel<16, SW, SPW, 8, SEG>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
            else
                hipLaunchKernelGGL((mfma_split_kernel<16, SW, SPW, 4, SEG>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
            return hipGetLastError();
        }
    }
    const size_t lds = (size_t)nks * (SW ? 2 : 1) * (MT / 16) * 4 * 65 * 4;
    hipLaunchKernelGGL((mfma_split_kernel<MT, SW, SPW, 0, SEG>), dim3((unsigned)tiles), dim3(64 * nks), lds, s, a);
    return hipGetLastError();
}

template <int MT, bool SW, int SPW>
hipError_t launch_mfma_split_one(const ProjArgs& a, hipStream_t s)
{
    if constexpr (!SW) {
        if (a.nseg > 1) return launch_mfma_split_seg<MT, SW, SPW, true>(a, s);
    }
    return launch_mfma_split_seg<MT, SW, SPW, false>(a, s);
}

template <int MT, bool SW>
hipError_t launch_mfma_split_mt(const ProjArgs& a, hipStream_t s)
{
    switch (mfma_split_spw(a.K, SW)) {
        case 2: return launch_mfma_split_one<MT, SW, 2>(a, s);
        case 4: return launch_mfma_split_one<MT, SW, 4>(a, s);
        case 6: return launch_mfma_split_one<MT, SW, 6>(a, s);
        case 8:
            if constexpr (!SW) return launch_mfma_split_one<MT, SW, 8>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <bool SW>
hipError_t launch_mfma_split_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.MT) {
        case 16: return launch_mfma_split_mt<16, SW>(a, s);
        case 32: return launch_mfma_split_mt<32, SW>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
