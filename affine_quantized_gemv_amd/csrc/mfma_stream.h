// Persistent matrix-core streaming kernel for large-N dense projections and
// fused SwiGLU at M = 9..32 (M padded to 16 or 32) on gfx950.
//
// y^T[N, M] = W[N, K] . x^T[K, M] with v_mfma_f32_16x16x32_bf16 (operand
// layouts as in mfma_kernel.h).  A row tile is 16 rows of W; a wavefront
// walks its tile's K/32 k-steps, each one MFMA per 16-column block of x^T,
// and keeps a ring of D k-steps of weights in flight across tile boundaries.
//
//   * A operands are read two k-steps (64 k, 128 bytes per row) at a time
//     with two buffer loads that each cover whole 128-byte lines: the first
//     reads rows 0..7 of the tile, the second rows 8..15; in each 16-lane
//     group g, lanes 0..7 take the 16-byte piece g of their row and lanes
//     8..15 the piece 4 + g.  One v_cndmask with a row_ror:8 DPP operand per
//     dword then forms the two MFMA A operands (all 16 rows, pieces 0..3 for
//     the first k-step, 4..7 for the second).  (A layout where each load
//     instruction covered 64 bytes of 16 rows measured ~25% slower.)  The
//     loads go through a wave-uniform per-tile descriptor; the k-block and
//     row-half offsets are uniform scalar offsets, so loads cost no vector
//     arithmetic.  Rows past N read as zero (outside the descriptor's range).
//   * x^T is staged once per workgroup in LDS in fragment order (for k-step s
//     and column block b the 64 lanes' 16-byte B operands are contiguous).
//   * Row tiles are dealt round-robin to all resident wavefronts, as in the
//     VALU streaming kernels; steady-state loads are unconditional and no
//     global store happens inside the loop; each tile's 16 x MT outputs are
//     staged in LDS and written after the loop.
//   * Each output is one chain of MFMAs over k in ascending order, the same
//     for every M the kernel serves (row independence within the path).
//
// Shapes and fused up/gate SwiGLU: AstrAI decode_linear_benchmark.md (commit
// message; M = 1..32 decode shapes and the LM head).
#pragma once
#include <atomic>

#include "mfma_kernel.h"
#include "piece_kernel.h"

namespace aqg {
namespace detail {

constexpr int kMfmaStreamThreads = 512;
constexpr size_t kMfmaStreamLdsMax = 160 * 1024;

template <int MT, bool SWIGLU, int D>
__global__ void __launch_bounds__(kMfmaStreamThreads) mfma_stream_kernel(ProjArgs a)
{
    extern __shared__ u32x4_t lds_m4[];
    constexpr int NB = MT / 16;          // 16-column blocks of x^T
    constexpr int S = SWIGLU ? 2 : 1;    // weight streams
    constexpr int NW = kMfmaStreamThreads / 64;
    constexpr int PER_TILE = 16 * MT;    // staged outputs per tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;             // k sub-block (A, B) / row quad (D)
    const int r = lane & 15;             // A row / B and D column
    const int KS = a.K / 32;             // k-steps per row
    const int KP = a.K / 64;             // k-step pairs per row
    const int64_t row_bytes = (int64_t)a.K * 2;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    const int64_t CT = a.tpw;
    const int64_t ST = (T + CT - 1) / CT;
    const int64_t W = (int64_t)gridDim.x * NW;
    const int64_t wg = (int64_t)blockIdx.x * NW + wave;
    int64_t my_tiles = 0;
    if (wg < ST) {
        const int64_t nst = (ST - 1 - wg) / W + 1;
        my_tiles = nst * CT;
        if ((ST - 1 - wg) % W == 0) my_tiles -= ST * CT - T;
    }

    u32x4_t* xb = lds_m4;                                                    // [s][b][lane]
    float* obuf = reinterpret_cast<float*>(lds_m4 + (size_t)KS * NB * 64) + (size_t)wave * a.tmax * PER_TILE;

    // ---- ring of D k-step pairs: slot d holds the two loads of one pair
    u32x4_t wa[D][S][2];
    int64_t f_tile = wg * CT;            // tile being fetched (wave-uniform)
    int f_c = 0;                         // its index within the super-tile
    int f_p = 0;                         // its k-step pair
    const int h = lane & 15;
    const uint32_t voff = (uint32_t)((h & 7) * row_bytes + 16 * ((h < 8 ? 0 : 4) + c));
    // rows 8..15: the row offset goes in the vector offset, which is the
    // part of the address the buffer range check covers
    const uint32_t voff_hi = voff + (uint32_t)(8 * row_bytes);
    auto fetch = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        const int64_t n0 = f_tile * 16;
        const int64_t bytes = (a.N - n0) * row_bytes;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const __amdgpu_buffer_rsrc_t rs =
                tile_rsrc(static_cast<const char*>(s == 0 ? a.w0 : a.w1) + n0 * row_bytes, bytes);
            wa[d][s][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 128 * f_p, kLoadNT));
            wa[d][s][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff_hi, 128 * f_p, kLoadNT));
        }
        // advance (tile, pair) without branches: wave-uniform selects
        const bool wrap = f_p + 1 == KP;
        const bool stw = wrap && f_c + 1 == CT;
        f_p = wrap ? 0 : f_p + 1;
        f_c = wrap ? (stw ? 0 : f_c + 1) : f_c;
        f_tile += wrap ? (stw ? (W - 1) * CT + 1 : 1) : 0;
    };
    // the two A operands of a pair: lanes 8..15 of each 16-lane group swap
    // halves across the two loads (rotate by 8 within the group)
    const bool hi8 = (lane & 8) != 0;
    auto a_ops = [&](const u32x4_t& l0, const u32x4_t& l1, u32x4_t& s0, u32x4_t& s1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0[i], 0x128, 0xF, 0xF, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1[i], 0x128, 0xF, 0xF, false);
            s0[i] = hi8 ? r1 : l0[i];
            s1[i] = hi8 ? l1[i] : r0;
        }
    };

    f32x4_t acc[S][NB];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int c_s = 0;                         // k-step pair being consumed
    int ti = 0;                          // tiles finished by this wavefront

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        u32x4_t A[S][2];
#pragma unroll
        for (int s = 0; s < S; ++s) a_ops(wa[d][s][0], wa[d][s][1], A[s][0], A[s][1]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const u32x4_t xv = xb[((2 * c_s + t) * NB + b) * 64 + lane];
#pragma unroll
                for (int s = 0; s < S; ++s) acc[s][b] = mfma16x16x32(A[s][t], xv, acc[s][b]);
            }
        if (++c_s == KP) {
            // end of a row tile: lane holds rows 4c..4c+3 of column r of each
            // column block; stage them (fp32), then reset
            c_s = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = acc[0][b][i];
                    if constexpr (SWIGLU) {
                        const float u = acc[1][b][i];
                        v = (v / (1.0f + __expf(-v))) * u;
                    }
                    obuf[ti * PER_TILE + (4 * c + i) * MT + 16 * b + r] = v;
                }
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ++ti;
        }
    };

    // prologue: D k-steps (past the wavefront's share they read zeros or
    // valid rows and are never consumed), then stage x^T
    static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(Dd); });
    // x^T staging, 8 loads in flight per thread before their stores
    constexpr int XB = 8;
    const int ntask = KS * NB * 64;
    for (int t0 = threadIdx.x; t0 < ntask; t0 += XB * kMfmaStreamThreads) {
        u32x4_t v[XB];
#pragma unroll
        for (int i = 0; i < XB; ++i) {
            const int t = t0 + i * kMfmaStreamThreads;
            const int l = t & 63;
            const int sb = t >> 6;       // s * NB + b
            const int s = sb / NB, b = sb - s * NB;
            const int m = 16 * b + (l & 15);
            v[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (t < ntask && m < a.M)
                v[i] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)m * a.K + 32 * s + 8 * (l >> 4));
        }
#pragma unroll
        for (int i = 0; i < XB; ++i) {
            const int t = t0 + i * kMfmaStreamThreads;
            if (t < ntask) xb[t] = v[i];
        }
    }
    // Every load issued so far is complete here (the x loads were issued
    // after the weights, and loads complete in order); saying so explicitly
    // keeps the compiler from carrying a possibly-pending staging load into
    // the loop, where it would wait for all loads in flight every iteration.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (my_tiles == 0) return;

    const int64_t nitems = my_tiles * KP;
    int64_t base = 0;
    for (; base + 2 * D <= nitems; base += D) {          // steady state
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            consume(Dd);
            fetch(Dd);
            // keep each slot's loads right after its own arithmetic: left
            // free, the scheduler moves them and the register assignment
            // around the loop then waits for every load in flight
            // (vmcnt(0)) at the top of each iteration
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    for (; base < nitems; base += D) {                   // drain
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int d = decltype(Dd)::value;
            if (base + d < nitems) {
                consume(Dd);
                if (base + d + D < nitems) fetch(Dd);
            }
        });
    }

    // write out: value v of the wavefront's list is tile v / (16*MT), row
    // (v / MT) % 16 of the tile, output row m = v % MT
    for (int v = lane; v < ti * PER_TILE; v += 64) {
        const int t2 = v / PER_TILE;
        const int rem = v % PER_TILE;
        const int m = rem % MT;
        const int64_t tile = (wg + (int64_t)(t2 / CT) * W) * CT + t2 % CT;
        const int64_t n = tile * 16 + rem / MT;
        if (m < a.M && n < a.N) {
            const float val = obuf[v];
            const size_t o = (size_t)m * a.N + n;
            if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = val;
            else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(val);
        }
    }
}

// LDS bytes of one workgroup: x^T fragments for the whole K plus the output
// staging of `tmax` tiles per wavefront.
inline size_t mfma_stream_lds_bytes(int MT, int K, int64_t tmax)
{
    return (size_t)(K / 32) * (MT / 16) * 64 * 16 + (size_t)(kMfmaStreamThreads / 64) * tmax * 16 * MT * 4;
}

// Depth (k-step pairs, 2 KB per weight stream, in flight per wavefront):
// on the 100000 x 1536 LM head, 3 measured ~8% faster than 4 at M = 32 and
// the same at M = 16 (more bytes in flight than that slow the stream down).
constexpr int kMfmaStreamDepth = 3;

template <int MT, bool SW>
hipError_t launch_mfma_stream_one(const ProjArgs& a, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&mfma_stream_kernel<MT, SW, kMfmaStreamDepth>);
    {
        hipError_t e = raise_lds_limit(fn, kMfmaStreamLdsMax);
        if (e != hipSuccess) return e;
    }
    int cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    constexpr int NW = kMfmaStreamThreads / 64;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    const int64_t ct = 1;
    const int64_t st = T;
    int64_t waves = st, tmax = 0;
    size_t lds = 0;
    for (int round = 0; round < 3; ++round) {
        tmax = ((st + waves - 1) / waves) * ct;
        lds = mfma_stream_lds_bytes(MT, a.K, tmax);
        if (lds > kMfmaStreamLdsMax) return hipErrorInvalidValue;
        int bpc = 0;
        e = occupancy(bpc, fn, kMfmaStreamThreads, lds);
        if (e != hipSuccess) return e;
        if (bpc < 1) bpc = 1;
        int64_t w = (int64_t)bpc * cus * NW;
        if (w > st) w = st;
        if (w == waves && round > 0) break;
        waves = w;
    }
    const int blocks = (int)((waves + NW - 1) / NW);
    tmax = ((st + (int64_t)blocks * NW - 1) / ((int64_t)blocks * NW)) * ct;
    lds = mfma_stream_lds_bytes(MT, a.K, tmax);
    if (lds > kMfmaStreamLdsMax) return hipErrorInvalidValue;
    ProjArgs a2 = a;
    a2.tpw = ct;
    a2.tmax = tmax;
    hipLaunchKernelGGL((mfma_stream_kernel<MT, SW, kMfmaStreamDepth>), dim3(blocks), dim3(kMfmaStreamThreads), lds, s, a2);
    return hipGetLastError();
}

template <bool SW>
hipError_t launch_mfma_stream_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.MT) {
        case 16: return launch_mfma_stream_one<16, SW>(a, s);
        case 32: return launch_mfma_stream_one<32, SW>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
