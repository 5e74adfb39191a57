// Persistent streaming kernel for M <= 8 (VALU path) on gfx950.
//
// Same arithmetic as proj_kernel (unit_mac), organised for bandwidth:
//   * x (all M rows, the whole K) is staged once per workgroup and stays
//     resident for the whole launch -- in LDS, or, for affine weights with
//     M <= 2 and one 64-code group per lane, directly in the lane's registers
//     (pre-scaled pair operands plus the group constants X and T);
//   * row tiles are grouped into super-tiles of ~4 KB of consecutive weights,
//     dealt round-robin to every resident wavefront: the device sweeps the
//     matrix as one moving window of contiguous reads (measured on MI355X:
//     such a sweep streams ~7 TB/s, several percent more than giving each
//     wavefront its own contiguous range), and wavefront loads differ by at
//     most one super-tile;
//   * a ring of D units of weights per lane stays in flight across row
//     boundaries, so HBM latency is paid once per wavefront, not per row;
//   * a row tile is G = 64 / 2^L rows: each 2^L-lane segment of the
//     wavefront owns one row; its lanes take the row's units round-robin and
//     are summed with the fixed segment tree at the end of the row.
// 2^L and the per-lane units depend on (bits, K) only, so every M computes
// each output the same way.
#pragma once
#include <atomic>

#include "piece_kernel.h"

namespace aqg {
namespace detail {

constexpr int kStreamThreads = 256;
constexpr size_t kStreamLdsMax = 160 * 1024;

// Units of weights in flight per lane: ~128 bytes for small M, fewer where
// the accumulators and x reads of a larger M need the registers.
template <int BITS, int MT> struct StreamDepth {
    static constexpr int D = BITS == 0 ? (MT <= 2 ? 8 : 4) : ((BITS <= 4 && MT <= 4) ? 4 : 2);
};

// One unit of weights (Geo<BITS>::NW words at byte offset voff + soff of a
// buffer) in 16-byte loads plus an 8-byte tail; non-temporal: weights are
// read once.
template <int BITS>
__device__ __forceinline__ void load_unit_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* w)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int NW = Geo<BITS>::NW;
    static_assert(NW % 2 == 0, "units are whole 8-byte pieces");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, kLoadNT));
        w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    if constexpr (NW % 4 != 0) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff + 16 * (NW / 4), soff, kLoadNT));
        w[NW - 2] = v.x; w[NW - 1] = v.y;
    }
}

template <int BITS, int MT, bool SWIGLU, bool XREG, int D = StreamDepth<BITS, MT>::D>
__global__ void __launch_bounds__(kStreamThreads) stream_kernel(ProjArgs a)
{
    extern __shared__ uint4 lds_s4[];
    constexpr int S = SWIGLU ? 2 : 1;
    constexpr int UK = Geo<BITS>::UK;
    constexpr int NW = Geo<BITS>::NW;
    constexpr int NCH = Geo<BITS>::NCH;
    static_assert(!XREG || BITS != 0, "register-resident x is for affine weights");

    const int L = a.lpr_log2;
    const int LPR = 1 << L;
    const int G = 64 >> L;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar tile math
    const int slot = lane >> L;
    const int li = lane & (LPR - 1);
    const int U = a.K / UK;                                   // units per row
    const int upl = (U + LPR - 1) >> L;                       // unit slots per lane
    const int64_t T = ((int64_t)a.N + G - 1) / G;             // row tiles
    // Super-tiles of C consecutive row tiles go round-robin over all W
    // wavefronts: at any moment the wavefronts read a window of adjacent
    // super-tiles, each a contiguous stretch of the weights.
    const int64_t CT = a.tpw;                                 // tiles per super-tile
    const int64_t ST = (T + CT - 1) / CT;
    const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t wg = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    int64_t my_tiles = 0;
    if (wg < ST) {
        const int64_t nst = (ST - 1 - wg) / W + 1;
        my_tiles = nst * CT;
        if ((ST - 1 - wg) % W == 0) my_tiles -= ST * CT - T;  // this wave owns the last, partial one
    }
    const int64_t row_words = (BITS == 0) ? (int64_t)a.K / 2 : (int64_t)a.K * BITS / 32;
    const int gpr = a.K / 64;

    // ---- stream: items are (tile, unit slot j) in order; ring of D items.
    // In the steady-state loop every load is unconditional (indices clamped to
    // a valid unit; an idle lane re-reads a neighbour's address, which
    // coalesces) and nothing writes global memory, so the vector-memory wait
    // counts stay exact: consuming ring slot d waits for slot d's loads only,
    // never for the D-1 younger ones.  Finished outputs go to a lane-private
    // slice of LDS and are written out after the loop by the same lane.
    uint32_t wb[D][S][1][NW];
    // scales and biases stay raw bf16 in the ring and are widened when their
    // slot is consumed: widened at fetch time, the conversion is an early
    // use of the youngest loads, and the compiler then waits for every load
    // in flight (vmcnt(0)) once per ring turn
    uint16_t sr[D][S], br[D][S];
    int64_t f_tile = wg * CT;   // next item to fetch: tile, its index within
    int f_c = 0;                // the super-tile, and the unit slot
    int f_j = 0;
    // next tile of this wavefront: the next one in the super-tile, else the
    // first of the super-tile W further on (counters, no 64-bit division)
    auto next_tile = [&](int64_t t) __attribute__((always_inline)) {
        ++t;
        if (++f_c == CT) { f_c = 0; t += (W - 1) * CT; }
        return t;
    };
    // Loads go through a buffer descriptor per row tile (base and byte range
    // of the tile's rows, scalar) with loop-invariant lane offsets, so a fetch
    // costs scalar work only.  Rows past N fall outside the range and read as
    // zero; a lane slot past the row's last unit reads into the next row or
    // outside the range, and its contribution is zeroed by `live` below.
    const int64_t row_bytes = row_words * 4;
    const uint32_t wvo = (uint32_t)((int64_t)slot * row_bytes + (int64_t)li * NW * 4);
    [[maybe_unused]] const uint32_t svo = (uint32_t)((slot * gpr + li) * 2);
    auto fetch = [&](int d) __attribute__((always_inline)) {
        const int64_t n0 = f_tile * G;
        const int64_t rows = a.N - n0;
        const uint32_t uo = (uint32_t)(f_j * LPR);            // this slot's first unit
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const char* base = static_cast<const char*>(s == 0 ? a.w0 : a.w1);
            load_unit_buf<BITS>(tile_rsrc(base + n0 * row_bytes, rows * row_bytes), wvo, uo * NW * 4, wb[d][s][0]);
        }
        if constexpr (BITS != 0) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc((s == 0 ? a.scales : a.scales1) + n0 * gpr, rows * gpr * 2);
                const __amdgpu_buffer_rsrc_t rb = tile_rsrc((s == 0 ? a.biases : a.biases1) + n0 * gpr, rows * gpr * 2);
                sr[d][s] = __builtin_amdgcn_raw_buffer_load_b16(rs, svo, uo * 2, kLoadNT);
                br[d][s] = __builtin_amdgcn_raw_buffer_load_b16(rb, svo, uo * 2, kLoadNT);
            }
        }
        if (++f_j == upl) { f_j = 0; f_tile = next_tile(f_tile); }
    };
    // prologue: D items, unconditionally (past the end they are clamped,
    // harmless re-reads that are never consumed)
    auto prologue_fetch = [&]() __attribute__((always_inline)) {
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(decltype(Dd)::value); });
    };

    // ---- x: LDS (whole K) or registers (one group per lane)
    uint4* xp = lds_s4;
    float2* xc = reinterpret_cast<float2*>(lds_s4 + MT * NCH * U);
    uint32_t xq[XREG ? MT : 1][XREG ? PairPlan<(BITS ? BITS : 2)>::NP : 1];
    float xX[MT], xT[MT];
    if constexpr (XREG) {
        // Lane li's operands are those of group li (the same in every
        // wavefront), so the workgroup computes each group's once into LDS
        // (MT*U <= 128 tasks, one per thread) and every lane copies its own:
        // the operand arithmetic (~500 VALU instructions per group) is paid
        // once per workgroup instead of once per wavefront.  The x loads go
        // out first, then the first weight loads, then that arithmetic, so
        // it waits for x alone and overlaps the weights' latency.
        using St = Stager<BITS, MT>;
        const St st{a, 0, U, xp, xc};
        const int ntask = st.ntasks();
        const bool mine = (int)threadIdx.x < ntask;
        typename St::Regs xr = st.load(mine ? (int)threadIdx.x : ntask - 1);
        prologue_fetch();
        if (mine) st.store(threadIdx.x, xr);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool have = li < U;
            const int g = have ? li : 0;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint4 v = have ? xp[(m * NCH + c) * U + g] : make_uint4(0, 0, 0, 0);
                xq[m][4 * c] = v.x; xq[m][4 * c + 1] = v.y; xq[m][4 * c + 2] = v.z; xq[m][4 * c + 3] = v.w;
            }
            const float2 v = have ? xc[m * U + g] : make_float2(0.0f, 0.0f);
            xX[m] = v.x;
            xT[m] = v.y;
        }
    } else {
        using St = Stager<BITS, MT>;
        St st = [&] {
            if constexpr (BITS == 0) return St{a, 0, U, xp};
            else return St{a, 0, U, xp, xc};
        }();
        constexpr int XB = (BITS == 0) ? 8 : 1;
        const int ntask = st.ntasks();
        const int nthr = blockDim.x;
        for (int t0 = threadIdx.x; t0 < ntask; t0 += XB * nthr) {
            typename St::Regs xr[XB];
#pragma unroll
            for (int i = 0; i < XB; ++i)
                if (t0 + i * nthr < ntask) xr[i] = st.load(t0 + i * nthr);
#pragma unroll
            for (int i = 0; i < XB; ++i)
                if (t0 + i * nthr < ntask) st.store(t0 + i * nthr, xr[i]);
        }
        __syncthreads();
    }
    if (my_tiles == 0) return;

    // lane-private output staging: VPL values per tile (outputs m = li + v*LPR)
    constexpr int VPL_MAX = MT;
    const int VPL = (MT + LPR - 1) >> L;
    float* obuf = reinterpret_cast<float*>(lds_s4 + MT * NCH * U + ((BITS != 0) ? (MT * U + 1) / 2 : 0))
                  + (size_t)wave * a.tmax * 64 * VPL;
    (void)VPL_MAX;

    const int64_t nitems = my_tiles * upl;
    if constexpr (!XREG) prologue_fetch();

    float acc[S][1][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][0][m] = 0.0f;
    int c_j = 0;
    int ti = 0;                 // tiles finished by this wavefront

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        {
            {
                // A lane past the row's last unit computes a duplicate of unit
                // U-1 with zeroed weights (dense) or zeroed scale and bias
                // (affine), so its contribution is exactly 0 -- no branch.
                const int u0 = li + c_j * LPR;
                const bool live = u0 < U;
                const int u = live ? u0 : U - 1;
                [[maybe_unused]] float sb[S][1], bb[S][1];
                if constexpr (BITS == 0) {
#pragma unroll
                    for (int s = 0; s < S; ++s)
#pragma unroll
                        for (int i = 0; i < NW; ++i) wb[d][s][0][i] = live ? wb[d][s][0][i] : 0u;
                } else {
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        sb[s][0] = live ? bf16_to_f32(sr[d][s]) : 0.0f;
                        bb[s][0] = live ? bf16_to_f32(br[d][s]) : 0.0f;
                    }
                }
                {
                    if constexpr (XREG) {
                        using P = PairPlan<BITS>;
                        // same order as unit_mac: even/odd pairs of a chunk
                        // into two accumulators, d = d0 + d1
                        float dd[S][MT], de[S][MT];
#pragma unroll
                        for (int s = 0; s < S; ++s)
#pragma unroll
                            for (int m = 0; m < MT; ++m) dd[s][m] = de[s][m] = 0.0f;
                        static_for<0, NCH>([&](auto C) __attribute__((always_inline)) {
                            constexpr int c = decltype(C)::value;
#pragma unroll
                            for (int s = 0; s < S; ++s) {
                                const uint32_t p0 = P::template pair<4 * c + 0>(wb[d][s][0]);
                                const uint32_t p1 = P::template pair<4 * c + 1>(wb[d][s][0]);
                                const uint32_t p2 = P::template pair<4 * c + 2>(wb[d][s][0]);
                                const uint32_t p3 = P::template pair<4 * c + 3>(wb[d][s][0]);
#pragma unroll
                                for (int m = 0; m < MT; ++m) {
                                    float v0 = dd[s][m], v1 = de[s][m];
                                    v0 = dot2(p0, xq[m][4 * c + 0], v0);
                                    v1 = dot2(p1, xq[m][4 * c + 1], v1);
                                    v0 = dot2(p2, xq[m][4 * c + 2], v0);
                                    v1 = dot2(p3, xq[m][4 * c + 3], v1);
                                    dd[s][m] = v0;
                                    de[s][m] = v1;
                                }
                            }
#pragma unroll
                            for (int s = 0; s < S; ++s)
#pragma unroll
                                for (int m = 0; m < MT; ++m) { pin(dd[s][m]); pin(de[s][m]); }
                            code_fence();
                        });
#pragma unroll
                        for (int m = 0; m < MT; ++m)
#pragma unroll
                            for (int s = 0; s < S; ++s)
                                acc[s][0][m] = fmaf(sb[s][0], (dd[s][m] + de[s][m]) - xT[m],
                                                    fmaf(bb[s][0], xX[m], acc[s][0][m]));
                    } else {
                        unit_mac<BITS, MT, S, 1>(wb[d], sb, bb, xp, xc, U, u, acc);
                    }
                }
                if (++c_j == upl) {
                    // end of a row tile: segment sums, epilogue, stage, reset
                    c_j = 0;
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float v = segment_sum64(acc[0][0][m], L);
                        if constexpr (SWIGLU) {
                            const float u2 = segment_sum64(acc[1][0][m], L);
                            v = (v / (1.0f + __expf(-v))) * u2;
                        }
#pragma unroll
                        for (int s = 0; s < S; ++s) acc[s][0][m] = 0.0f;
                        // lane (m mod 2^L) of the segment owns output m
                        if ((m & (LPR - 1)) == li) obuf[((size_t)ti * VPL + (m >> L)) * 64 + lane] = v;
                    }
                    ++ti;
                }
            }
        }
    };

    int64_t base = 0;
    for (; base + 2 * D <= nitems; base += D) {         // steady state: no branches around memory ops
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            consume(Dd);
            fetch(decltype(Dd)::value);
            // keep each slot's loads right after its arithmetic, so a slot
            // waits for its own loads only
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    for (; base < nitems; base += D) {                  // drain
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int d = decltype(Dd)::value;
            if (base + d < nitems) {
                consume(Dd);
                if (base + d + D < nitems) fetch(d);
            }
        });
    }

    // write out the staged outputs (each lane reads back only its own values)
    for (int t2 = 0; t2 < ti; ++t2) {
        const int64_t tile = (wg + (int64_t)(t2 / CT) * W) * CT + t2 % CT;
        const int64_t n = tile * G + slot;
        for (int v = 0; v < VPL; ++v) {
            const int m = li + v * LPR;
            if (m < a.M && n < a.N) {
                const float val = obuf[((size_t)t2 * VPL + v) * 64 + lane];
                const size_t o = (size_t)m * a.N + n;
                if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = val;
                else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(val);
            }
        }
    }
}

// LDS bytes of one workgroup: the staged x (with x in registers, the operands
// the lanes copy from) plus the lane-private output staging for `tmax` tiles
// per wavefront.
template <int BITS, int MT, bool XREG>
size_t stream_lds_bytes(const LaunchCfg& c, int K, int64_t tmax)
{
    const int L = c.lpr_log2;
    const int vpl = (MT + (1 << L) - 1) >> L;
    const size_t out = (size_t)c.nwaves * tmax * 64 * vpl * 4;
    const int U = BITS == 0 ? K / 8 : K / 64;
    const size_t x16 = (size_t)MT * Geo<BITS>::NCH * U + (BITS != 0 ? ((size_t)MT * U + 1) / 2 : 0);
    return x16 * 16 + out;
}

template <int BITS, int MT, bool SW, bool XREG>
hipError_t launch_stream_one(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&stream_kernel<BITS, MT, SW, XREG>);
    {
        // allow up to 160 KB of dynamic LDS (gfx950 has 160 KB per CU); once
        hipError_t e = raise_lds_limit(fn, kStreamLdsMax);
        if (e != hipSuccess) return e;
    }
    int cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    const int L = c.lpr_log2;
    const int64_t G = 64 >> L;
    const int64_t T = ((int64_t)a.N + G - 1) / G;
    const int64_t row_bytes = BITS == 0 ? (int64_t)a.K * 2 : (int64_t)a.K * BITS / 8;
    int64_t ct = 4096 / (G * row_bytes);                      // ~4 KB super-tiles
    if (ct < 1) ct = 1;
    const int64_t st = (T + ct - 1) / ct;
    // Grid: every wavefront slot the device can hold at once (occupancy at this
    // LDS size; the output staging depends on the grid, so settle in 3 rounds).
    int64_t waves = st, tmax = 0;
    size_t lds = 0;
    for (int round = 0; round < 3; ++round) {
        tmax = ((st + waves - 1) / waves) * ct;
        lds = stream_lds_bytes<BITS, MT, XREG>(c, a.K, tmax);
        if (lds > kStreamLdsMax) return hipErrorInvalidValue;
        int bpc = 0;
        e = occupancy(bpc, fn, 64 * c.nwaves, lds);
        if (e != hipSuccess) return e;
        if (bpc < 1) bpc = 1;
        int64_t w = (int64_t)bpc * cus * c.nwaves;
        if (w > st) w = st;
        if (w == waves && round > 0) break;
        waves = w;
    }
    tmax = ((st + waves - 1) / waves) * ct;
    lds = stream_lds_bytes<BITS, MT, XREG>(c, a.K, tmax);
    ProjArgs a2 = a;
    a2.tpw = ct;
    a2.tmax = tmax;
    const int blocks = (int)((waves + c.nwaves - 1) / c.nwaves);
    hipLaunchKernelGGL((stream_kernel<BITS, MT, SW, XREG>), dim3(blocks), dim3(64 * c.nwaves), lds, s, a2);
    return hipGetLastError();
}

template <int BITS, bool SW>
hipError_t launch_stream_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if constexpr (BITS != 0) {
        if (c.xreg) {
            if (c.MT == 1) return launch_stream_one<BITS, 1, SW, true>(a, c, s);
            if constexpr (BITS != 8)
                if (c.MT == 2) return launch_stream_one<BITS, 2, SW, true>(a, c, s);
            return hipErrorInvalidValue;
        }
    }
    switch (c.MT) {
        case 1: return launch_stream_one<BITS, 1, SW, false>(a, c, s);
        case 2: return launch_stream_one<BITS, 2, SW, false>(a, c, s);
        case 4: return launch_stream_one<BITS, 4, SW, false>(a, c, s);
        case 8: return launch_stream_one<BITS, 8, SW, false>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
