// Persistent streaming kernel with 16-byte pieces, M <= 8, for dense bf16
// weights and affine codes of width 2, 4 and 8 (whose codes never straddle a
// 16-byte boundary).
//
// Every load instruction of a wavefront reads whole 128-byte lines: the 2^L
// lanes of a row segment each load one 16-byte piece, lane li taking pieces
// li, li + 2^L, li + 2*2^L, ... of the row, so one instruction covers 2^L * 16
// contiguous bytes of each of the wavefront's G = 64 / 2^L rows (measured on
// MI355X, reads in which each instruction covers only part of its lines --
// one lane owning a whole 32- or 64-byte group -- stream 20-45% slower).
//
// A piece is 8 bf16 weights (dense) or 128/b codes: half a group at b = 4, a
// quarter at b = 8, a whole group at b = 2.  Its arithmetic is the factored
// form of the affine product on the piece: d = sum of dot2(code pair operand,
// pre-scaled x pair) over the piece's pair plan, acc += scale*(d - T) +
// bias*X with the piece's own T and X; summed over the pieces of a group this
// is the group's exact sum_k x*(scale*q + bias) up to fp32 rounding.
//
// Each lane's pieces sit at fixed k offsets of every row, so their x operands
// (all M rows) are computed once and kept in registers when they fit, else
// staged in LDS in the same form by the same routine; both give bit-identical
// results.  The rest follows the streaming kernel: super-tiles of consecutive
// row tiles dealt round-robin to all resident wavefronts, a ring of loads
// that stays in flight across row boundaries with unconditional (clamped)
// loads in the steady state, outputs staged in LDS and written at the end.
// J = pieces per lane per row is a compile-time constant, so every ring slot
// knows its piece (and its x registers) statically.
#pragma once
#include <atomic>

#include "proj_kernel.h"

namespace aqg {
namespace detail {

constexpr int kPieceThreads = 256;
constexpr size_t kPieceLdsMax = 160 * 1024;
constexpr int kPieceXregBudget = 128;   // x-operand registers per lane

template <int BITS> struct PieceGeo {
    using Plan = PiecePlan<BITS>;
    static constexpr int KPP = 128 / BITS;          // k per piece
    static constexpr int NPP = Plan::NP;            // bf16x2 x operands per (m, piece)
    static constexpr int PPG = 64 / KPP;            // pieces per group
};
template <> struct PieceGeo<0> {
    static constexpr int KPP = 8;
    static constexpr int NPP = 4;
    static constexpr int PPG = 1;
};

template <int BITS, int MT, int J>
constexpr bool piece_xreg_ok() { return PieceGeo<BITS>::NPP * J * MT <= kPieceXregBudget; }

// Row tiles in flight per wavefront: about 4 pieces per lane, at least 2 rows
// when a row has fewer than 4 pieces per lane.
template <int J> struct PieceDepth {
    static constexpr int RD = J >= 4 ? 1 : (J >= 2 ? 2 : 4);
};

// x operands of one piece for one row m: dense, the 8 bf16 as they are;
// affine, the piece plan's pre-scaled pairs plus X and T.
template <int BITS>
__device__ __forceinline__ void piece_x(const uint16_t* __restrict__ xrow, bool have,
                                        uint32_t (&xq)[PieceGeo<BITS>::NPP], float& X, float& T)
{
    constexpr int KPP = PieceGeo<BITS>::KPP;
    uint32_t xw[KPP / 2];
    const uint4* src = reinterpret_cast<const uint4*>(xrow);
#pragma unroll
    for (int i = 0; i < KPP / 8; ++i) {
        const uint4 v = have ? src[i] : make_uint4(0, 0, 0, 0);
        xw[4 * i] = v.x; xw[4 * i + 1] = v.y; xw[4 * i + 2] = v.z; xw[4 * i + 3] = v.w;
    }
    if constexpr (BITS == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[i] = xw[i];
        X = T = 0.0f;
    } else {
        plan_x_operands<PiecePlan<BITS>, KPP / 2>(xw, xq, X, T);
    }
}

template <int BITS, int MT, bool SWIGLU, bool XREG, int J, int RD = PieceDepth<J>::RD>
__global__ void __launch_bounds__(kPieceThreads) piece_kernel(ProjArgs a)
{
    extern __shared__ uint4 lds_p4[];
    constexpr int S = SWIGLU ? 2 : 1;
    using PG = PieceGeo<BITS>;
    constexpr int KPP = PG::KPP;
    constexpr int NPP = PG::NPP;
    constexpr int NCHP = NPP / 4;                 // uint4 chunks of x operands per (m, piece)
    constexpr int D = RD * J;                     // ring slots (pieces in flight per lane)
    static_assert(!SWIGLU || BITS == 0, "the fused SwiGLU takes dense weights");

    const int L = a.lpr_log2;
    const int P = 1 << L;
    const int G = 64 >> L;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane >> L;
    const int li = lane & (P - 1);
    const int PR = a.K / KPP;                                 // pieces per row
    const bool ragged = J * P != PR;                          // last piece slot partly empty
    const int64_t T = ((int64_t)a.N + G - 1) / G;             // row tiles
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
    const int64_t row_words = (int64_t)PR * 4;
    const int gpr = a.K / 64;

    // ---- x operands: registers or LDS (whole K, all MT rows)
    uint4* xp = lds_p4;                                                   // [m][chunk][piece]
    float2* xc = reinterpret_cast<float2*>(lds_p4 + (size_t)MT * NCHP * PR);  // [m][piece] (X, T)
    uint32_t xq[XREG ? J : 1][XREG ? MT : 1][NPP];
    float xX[XREG ? J : 1][XREG ? MT : 1], xT[XREG ? J : 1][XREG ? MT : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int p = li + P * j;
                const bool have = m < a.M && p < PR;
                piece_x<BITS>(a.x + (size_t)m * a.K + (size_t)(have ? p : 0) * KPP, have,
                              xq[j][m], xX[j][m], xT[j][m]);
            }
    } else {
        const int ntask = MT * PR;
        for (int t = threadIdx.x; t < ntask; t += blockDim.x) {
            const int m = t / PR, p = t - m * PR;
            uint32_t q[NPP];
            float X, Tc;
            piece_x<BITS>(a.x + (size_t)m * a.K + (size_t)p * KPP, m < a.M, q, X, Tc);
#pragma unroll
            for (int c = 0; c < NCHP; ++c)
                xp[((size_t)m * NCHP + c) * PR + p] = make_uint4(q[4 * c], q[4 * c + 1], q[4 * c + 2], q[4 * c + 3]);
            if constexpr (BITS != 0) xc[(size_t)m * PR + p] = make_float2(X, Tc);
        }
        __syncthreads();
    }
    if (my_tiles == 0) return;

    // ---- output staging: G*MT fp32 per finished tile, wavefront-private
    const int per_tile = G * MT;
    float* obuf = reinterpret_cast<float*>(
                      XREG ? lds_p4
                           : lds_p4 + (size_t)MT * NCHP * PR + (BITS != 0 ? ((size_t)MT * PR + 1) / 2 : 0))
                  + (size_t)wave * a.tmax * per_tile;

    // ---- ring of D = RD*J slots; slot d holds piece j = d % J of a row tile.
    // Loads in the steady state are unconditional (rows and pieces clamped to
    // valid addresses; clamped values are never used) and nothing is stored
    // to global memory inside the loop, so every wait is for one slot's loads.
    uint32_t wb[D][S][4];
    [[maybe_unused]] float sb[D], bb[D];
    int64_t f_tile = wg * CT;
    int f_c = 0;
    auto next_tile = [&](int64_t t) __attribute__((always_inline)) {
        ++t;
        if (++f_c == CT) { f_c = 0; t += (W - 1) * CT; }
        return t;
    };
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    auto fetch = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        constexpr int j = d % J;
        int p = li + P * j;
        if (p >= PR) p = PR - 1;
        int64_t n = f_tile * G + slot;
        if (n >= a.N) n = a.N - 1;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint32_t* base = reinterpret_cast<const uint32_t*>(s == 0 ? a.w0 : a.w1);
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + n * row_words + (int64_t)p * 4));
            wb[d][s][0] = v.x; wb[d][s][1] = v.y; wb[d][s][2] = v.z; wb[d][s][3] = v.w;
        }
        if constexpr (BITS != 0) {
            const int g = p / PG::PPG;
            sb[d] = bf16_to_f32(a.scales[n * gpr + g]);
            bb[d] = bf16_to_f32(a.biases[n * gpr + g]);
        }
        if constexpr (j == J - 1) f_tile = next_tile(f_tile);
    };

    float acc[S][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
    int ti = 0;                 // tiles finished by this wavefront

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        constexpr int j = d % J;
        // x in LDS is loop-invariant; the fence keeps its reads here instead
        // of letting them be hoisted out of the loop into registers
        if constexpr (!XREG) code_fence();
        const int p0 = li + P * j;
        const bool live = p0 < PR;
        const int p = live ? p0 : PR - 1;
        // An empty piece slot (the row's last, ragged slot) contributes
        // exactly 0: zeroed weights (dense) or zeroed scale and bias (affine).
        if (ragged) {
            if constexpr (BITS == 0) {
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i) wb[d][s][i] = live ? wb[d][s][i] : 0u;
            } else {
                sb[d] = live ? sb[d] : 0.0f;
                bb[d] = live ? bb[d] : 0.0f;
            }
        }
        if constexpr (BITS == 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint32_t xv[4];
                if constexpr (XREG) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[i] = xq[j][m][i];
                } else {
                    const uint4 v = xp[(size_t)m * PR + p];
                    xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
                }
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[s][m] = dot2(wb[d][s][i], xv[i], acc[s][m]);
            }
        } else {
            using Plan = PiecePlan<BITS>;
            // pairs 4c+0, 4c+2 into one accumulator, 4c+1, 4c+3 into the other
            float dd[MT], de[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) dd[m] = de[m] = 0.0f;
            static_for<0, NCHP>([&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value;
                const uint32_t q0 = Plan::template pair<4 * c + 0>(wb[d][0]);
                const uint32_t q1 = Plan::template pair<4 * c + 1>(wb[d][0]);
                const uint32_t q2 = Plan::template pair<4 * c + 2>(wb[d][0]);
                const uint32_t q3 = Plan::template pair<4 * c + 3>(wb[d][0]);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    uint32_t x0, x1, x2, x3;
                    if constexpr (XREG) {
                        x0 = xq[j][m][4 * c]; x1 = xq[j][m][4 * c + 1];
                        x2 = xq[j][m][4 * c + 2]; x3 = xq[j][m][4 * c + 3];
                    } else {
                        const uint4 v = xp[((size_t)m * NCHP + c) * PR + p];
                        x0 = v.x; x1 = v.y; x2 = v.z; x3 = v.w;
                    }
                    float v0 = dd[m], v1 = de[m];
                    v0 = dot2(q0, x0, v0);
                    v1 = dot2(q1, x1, v1);
                    v0 = dot2(q2, x2, v0);
                    v1 = dot2(q3, x3, v1);
                    dd[m] = v0;
                    de[m] = v1;
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) { pin(dd[m]); pin(de[m]); }
                code_fence();
            });
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float X, Tc;
                if constexpr (XREG) {
                    X = xX[j][m];
                    Tc = xT[j][m];
                } else {
                    const float2 v = xc[(size_t)m * PR + p];
                    X = v.x;
                    Tc = v.y;
                }
                acc[0][m] = fmaf(sb[d], (dd[m] + de[m]) - Tc, fmaf(bb[d], X, acc[0][m]));
            }
        }
        if constexpr (j == J - 1) {
            // end of a row tile: segment sums, epilogue, stage, reset
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float v = segment_sum64(acc[0][m], L);
                if constexpr (SWIGLU) {
                    const float u = segment_sum64(acc[1][m], L);
                    v = (v / (1.0f + __expf(-v))) * u;
                }
#pragma unroll
                for (int s = 0; s < S; ++s) acc[s][m] = 0.0f;
                if (li == (m & (P - 1))) obuf[(size_t)ti * per_tile + slot * MT + m] = v;
            }
            ++ti;
        }
    };

    // prologue: RD rows, unconditionally
    static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(Dd); });
    int64_t bt = 0;
    for (; bt + 2 * RD <= my_tiles; bt += RD) {          // steady state
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            consume(Dd);
            fetch(Dd);
        });
    }
    for (; bt < my_tiles; bt += RD) {                   // drain
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int r = decltype(Dd)::value / J;
            if (bt + r < my_tiles) {
                consume(Dd);
                if (bt + r + RD < my_tiles) fetch(Dd);
            }
        });
    }

    // write out the staged outputs: value v of the wavefront's list is tile
    // v / (G*MT), row slot (v / MT) % G, output row m = v % MT
    const int lg_pt = __builtin_ctz(per_tile);
    const int lg_mt = __builtin_ctz(MT);
    for (int v = lane; v < ti * per_tile; v += 64) {
        const int t2 = v >> lg_pt;
        const int r = v & (per_tile - 1);
        const int m = r & (MT - 1);
        const int64_t tile = (wg + (int64_t)(t2 / CT) * W) * CT + t2 % CT;
        const int64_t n = tile * G + (r >> lg_mt);
        if (m < a.M && n < a.N) {
            const float val = obuf[v];
            const size_t o = (size_t)m * a.N + n;
            if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = val;
            else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(val);
        }
    }
}

// LDS bytes of one workgroup of `nwaves` wavefronts: staged x (none when x is
// in registers) plus the output staging for `tmax` tiles per wavefront.
template <int BITS>
size_t piece_lds_bytes(int MT, bool xreg, int L, int nwaves, int K, int64_t tmax)
{
    const int G = 64 >> L;
    const size_t out = (size_t)nwaves * tmax * G * MT * 4;
    if (xreg) return out;
    const int PR = K / PieceGeo<BITS>::KPP;
    const size_t x16 = (size_t)MT * (PieceGeo<BITS>::NPP / 4) * PR + (BITS != 0 ? ((size_t)MT * PR + 1) / 2 : 0);
    return x16 * 16 + out;
}

template <int BITS, int MT, bool SW, bool XREG, int J>
hipError_t launch_piece_one(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&piece_kernel<BITS, MT, SW, XREG, J>);
    {
        static std::atomic<int> raised{0};
        if (!raised.load(std::memory_order_acquire)) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPieceLdsMax);
            if (e != hipSuccess) return e;
            raised.store(1, std::memory_order_release);
        }
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int L = c.lpr_log2;
    const int64_t G = 64 >> L;
    const int64_t T = ((int64_t)a.N + G - 1) / G;
    const int64_t row_bytes = BITS == 0 ? (int64_t)a.K * 2 : (int64_t)a.K * BITS / 8;
    int64_t ct = 4096 / (G * row_bytes);                      // ~4 KB super-tiles
    if (ct < 1) ct = 1;
    const int64_t st = (T + ct - 1) / ct;
    // Grid: every wavefront slot the device holds at once at this LDS size
    // (the output staging depends on the grid: settle in a few rounds).
    int64_t waves = st, tmax = 0;
    size_t lds = 0;
    for (int round = 0; round < 3; ++round) {
        tmax = ((st + waves - 1) / waves) * ct;
        lds = piece_lds_bytes<BITS>(MT, XREG, L, c.nwaves, a.K, tmax);
        if (lds > kPieceLdsMax) return hipErrorInvalidValue;
        int bpc = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, 64 * c.nwaves, lds);
        if (e != hipSuccess) return e;
        if (bpc < 1) bpc = 1;
        int64_t w = (int64_t)bpc * cus * c.nwaves;
        if (w > st) w = st;
        if (w == waves && round > 0) break;
        waves = w;
    }
    tmax = ((st + waves - 1) / waves) * ct;
    lds = piece_lds_bytes<BITS>(MT, XREG, L, c.nwaves, a.K, tmax);
    if (lds > kPieceLdsMax) return hipErrorInvalidValue;
    ProjArgs a2 = a;
    a2.tpw = ct;
    a2.tmax = tmax;
    const int blocks = (int)((waves + c.nwaves - 1) / c.nwaves);
    hipLaunchKernelGGL((piece_kernel<BITS, MT, SW, XREG, J>), dim3(blocks), dim3(64 * c.nwaves), lds, s, a2);
    return hipGetLastError();
}

template <int BITS, int MT, bool SW, int J>
hipError_t launch_piece_mt(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (c.xreg) {
        if constexpr (piece_xreg_ok<BITS, MT, J>()) return launch_piece_one<BITS, MT, SW, true, J>(a, c, s);
        else return hipErrorInvalidValue;
    }
    return launch_piece_one<BITS, MT, SW, false, J>(a, c, s);
}

template <int BITS, bool SW, int J>
hipError_t launch_piece_j(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.MT) {
        case 1: return launch_piece_mt<BITS, 1, SW, J>(a, c, s);
        case 2: return launch_piece_mt<BITS, 2, SW, J>(a, c, s);
        case 4: return launch_piece_mt<BITS, 4, SW, J>(a, c, s);
        case 8: return launch_piece_mt<BITS, 8, SW, J>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

template <int BITS, bool SW>
hipError_t launch_piece_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.pieces_per_lane) {
        case 1: return launch_piece_j<BITS, SW, 1>(a, c, s);
        case 2: return launch_piece_j<BITS, SW, 2>(a, c, s);
        case 3: return launch_piece_j<BITS, SW, 3>(a, c, s);
        case 4: return launch_piece_j<BITS, SW, 4>(a, c, s);
        case 8: return launch_piece_j<BITS, SW, 8>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
