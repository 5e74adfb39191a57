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
// results.  A lane slot past the row's last piece (rows whose piece count is
// not a multiple of 2^L) gets zero x operands, which makes its contribution
// exactly zero without any masking.
//
// Weights, scales and biases are read with buffer loads: the row tile is
// wave-uniform, so its base address and byte range live in a scalar buffer
// descriptor, and each lane's offset into the tile is a loop-invariant 32-bit
// register.  Rows past N fall outside the descriptor's range and read as zero
// without touching memory.  A tile's scales (and biases) are G*K/64 <= 64
// adjacent bf16: lane g loads the tile's group g (one 128-byte instruction
// per tile, range-checked to the exact byte), and each piece takes its
// group's value from that lane with ds_bpermute -- two narrow loads per piece
// measured 15% slower.  The rest follows the streaming kernel:
// super-tiles of consecutive row tiles dealt round-robin to the resident
// wavefronts, a ring of loads that stays in flight across row boundaries
// (steady-state loads are unconditional, nothing is stored to global memory
// in the loop, so each wait is for one slot's loads), outputs staged in LDS
// and written at the end.  L and J (pieces per lane per row) are compile-time
// constants, so the loop body has no branches besides the loop itself.
#pragma once
#include <atomic>

#include "argmax.h"
#include "proj_kernel.h"

namespace aqg {
namespace detail {

constexpr int kPieceThreads = 256;
constexpr size_t kPieceLdsMax = 160 * 1024;
// x-operand registers per lane above which x is staged in LDS instead
// (affine: with the unpack's registers, more measured slower than LDS)
template <int BITS> constexpr int piece_xreg_budget() { return BITS == 0 ? 128 : 64; }
// Resident wavefronts per CU: more were measured no faster (dense: 8 with
// ~3 KB in flight each; affine, with more arithmetic per byte: 24, and 20 at
// M = 1, where each wavefront's set-up is a larger share of its work: 4-bit
// 14336 x 4096 7.9 us at 16 or 20 against 8.7 us at 24 or 28, the 4-bit LM
// head 15.3 against 15.6 us).
template <int BITS, int MT> constexpr int piece_max_waves_per_cu() { return BITS == 0 ? 8 : MT == 1 ? 20 : 24; }
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kLoadNT = 2;                // non-temporal: weights are read once

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
constexpr bool piece_xreg_ok() { return PieceGeo<BITS>::NPP * J * MT <= piece_xreg_budget<BITS>(); }

// Row tiles in flight per wavefront (measured on the LM-head shapes): 2 while
// a lane has at most 3 pieces per row, 1 from 4 pieces, and 1 for dense
// M <= 2 and affine M = 1 (which instead run more wavefronts per CU).
template <int BITS, int J, int MT> struct PieceDepth {
    static constexpr int RD = J >= 4 ? 1 : ((BITS == 0 ? MT <= 2 : MT == 1) ? 1 : 2);
};

// x operands of one piece for one row m from its KPP x values (as bf16 pair
// words): dense, the 8 bf16 as they are; affine, the piece plan's pre-scaled
// pairs plus X and T.
template <int BITS>
__device__ __forceinline__ void piece_operands(const uint32_t (&xw)[PieceGeo<BITS>::KPP / 2],
                                               uint32_t (&xq)[PieceGeo<BITS>::NPP], float& X, float& T)
{
    if constexpr (BITS == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[i] = xw[i];
        X = T = 0.0f;
    } else {
        plan_x_operands<PiecePlan<BITS>, PieceGeo<BITS>::KPP / 2>(xw, xq, X, T);
    }
}

// The same from memory; have = false gives all zeros.
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
    piece_operands<BITS>(xw, xq, X, T);
}

// Buffer descriptor over `bytes` bytes from p (clamped to [0, 0x7FFFFFF0]).
// The clamp compares the two 32-bit halves: a signed 64-bit compare has no
// scalar form, so it would run on the vector unit in every stream loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int64_t bytes)
{
    // (an empty asm keeps the halves apart: recombined, they would become
    // that 64-bit compare again; the descriptor is wave-uniform, so is hi)
    int hi = __builtin_amdgcn_readfirstlane((int)(bytes >> 32));
    asm("" : "+s"(hi));
    const uint32_t lo = (uint32_t)bytes;
    const int n = hi < 0 ? 0 : ((hi > 0 || lo >= 0x7FFFFFF0u) ? 0x7FFFFFF0 : (int)lo);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, kBufferFlags);
}

// Buffer descriptor over n >= 0 bytes from p (n already within range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int n)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, kBufferFlags);
}

// min(max(rows, 0), g) for a wave-uniform row count, with 32-bit scalar
// compares on the two halves (see tile_rsrc).
__device__ __forceinline__ int rows_in_tile(int64_t rows, int g)
{
    int hi = __builtin_amdgcn_readfirstlane((int)(rows >> 32));
    asm("" : "+s"(hi));
    const uint32_t lo = (uint32_t)rows;
    return hi < 0 ? 0 : ((hi > 0 || lo >= (uint32_t)g) ? g : (int)lo);
}

// s_waitcnt immediate for lgkmcnt(0) alone (vmcnt and expcnt at their
// maximum, i.e. not waited for): gfx9-family encoding.
__host__ __device__ constexpr int waitcnt_lgkm0_only() { return 0xF | 0x70 | (3 << 14); }

// A workgroup barrier with no implied wait for loads in flight (the memory
// clobber keeps the compiler from moving LDS accesses across it).
__device__ __forceinline__ void piece_barrier() { asm volatile("s_barrier" ::: "memory"); }

// SEG: a multi-projection launch (row tiles looked up in the projection
// table); a separate instantiation, since the per-tile lookup's scalar work
// inside the stream loop measured ~15% slower on the 4-bit LM head.
template <int BITS, int MT, bool SWIGLU, bool XREG, int L, int J, bool SEG = false,
          int RD = PieceDepth<BITS, J, MT>::RD>
__global__ void __launch_bounds__(kPieceThreads) piece_kernel(ProjArgs a)
{
    extern __shared__ uint4 lds_p4[];
    constexpr int S = SWIGLU ? 2 : 1;
    using PG = PieceGeo<BITS>;
    constexpr int KPP = PG::KPP;
    constexpr int NPP = PG::NPP;
    constexpr int NCHP = NPP / 4;                 // uint4 chunks of x operands per (m, piece)
    constexpr int D = RD * J;                     // ring slots (pieces in flight per lane)
    constexpr int P = 1 << L;                     // lanes per row
    constexpr int G = 64 >> L;                    // rows per tile
    constexpr int PRP = J * P;                    // piece slots per row (>= pieces per row)
    constexpr int PER_TILE = G * MT;              // staged outputs per tile
    static_assert(L >= 2 && L <= 6, "segment of 4..64 lanes");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = lane >> L;
    const int li = lane & (P - 1);
    const int PR = a.K / KPP;                                 // pieces per row
    const int64_t row_bytes = (int64_t)PR * 16;
    const int gpr = a.K / 64;
    const int64_t T = ((int64_t)a.N + G - 1) / G;             // row tiles
    const int64_t CT = a.tpw;                                 // tiles per super-tile
    const int64_t ST = (T + CT - 1) / CT;
    const int64_t W = (int64_t)gridDim.x * (kPieceThreads / 64);
    const int64_t wg = (int64_t)blockIdx.x * (kPieceThreads / 64) + wave;
    int64_t my_tiles = 0;
    if (wg < ST) {
        const int64_t nst = (ST - 1 - wg) / W + 1;
        my_tiles = nst * CT;
        if ((ST - 1 - wg) % W == 0) my_tiles -= ST * CT - T;  // this wave owns the last, partial one
    }

    // ---- x operands: registers or LDS (PRP piece slots per row, zero past PR).
    // Their loads go out before the first weight loads and their arithmetic
    // after them (see the prologue), so the latencies overlap.
    uint4* xp = lds_p4;                                                   // [m][chunk][piece slot]
    float2* xc = reinterpret_cast<float2*>(lds_p4 + (size_t)MT * NCHP * PRP);  // [m][piece slot] (X, T)
    uint32_t xq[XREG ? J : 1][XREG ? MT : 1][NPP];
    float xX[XREG ? J : 1][XREG ? MT : 1], xT[XREG ? J : 1][XREG ? MT : 1];
    // The workgroup computes every (m, piece slot) operand once into LDS
    // (XB tasks per thread with their loads in flight together), then
    // synchronizes.  Affine operands take ~100 VALU instructions per piece,
    // so computing them per lane in every wavefront would delay the first
    // weights by microseconds.
    // `between` runs after the first round's x loads are issued and before
    // they are used: the prologue issues the first weight loads there, so the
    // operand arithmetic waits for x alone and overlaps the weights' latency,
    // and the closing barrier waits for the LDS writes only.  Without weights
    // in flight (`between` empty) it is a plain __syncthreads (a bare barrier
    // there let the compiler keep staged x in registers across the loop on
    // dense M = 8, 7.5 -> 9.4 us).
    auto stage_x = [&](auto&& between, auto Early) __attribute__((always_inline)) {
        constexpr int XB = BITS == 0 ? 8 : 2;
        constexpr int KW = KPP / 2;                     // x words per piece
        auto load_round = [&](int t0, uint32_t (&xw)[XB][KW]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kPieceThreads;
                const int m = t / PRP, p = t - m * PRP;
                const bool have = t < MT * PRP && m < a.M && p < PR;
                const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)(have ? m : 0) * a.K +
                                                                  (size_t)(have ? p : 0) * KPP);
#pragma unroll
                for (int w = 0; w < KW / 4; ++w) {
                    const uint4 v = have ? src[w] : make_uint4(0, 0, 0, 0);
                    xw[i][4 * w] = v.x; xw[i][4 * w + 1] = v.y; xw[i][4 * w + 2] = v.z; xw[i][4 * w + 3] = v.w;
                }
            }
        };
        auto store_round = [&](int t0, uint32_t (&xw)[XB][KW]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kPieceThreads;
                if (t >= MT * PRP) break;
                const int m = t / PRP, p = t - m * PRP;
                uint32_t q[NPP];
                float X, Tc;
                piece_operands<BITS>(xw[i], q, X, Tc);
#pragma unroll
                for (int c = 0; c < NCHP; ++c)
                    xp[(m * NCHP + c) * PRP + p] = make_uint4(q[4 * c], q[4 * c + 1], q[4 * c + 2], q[4 * c + 3]);
                if constexpr (BITS != 0) xc[m * PRP + p] = make_float2(X, Tc);
            }
        };
        if constexpr (decltype(Early)::value) {
            // one round (the caller checks): every thread, loads predicated
            uint32_t xw[XB][KW];
            load_round(threadIdx.x, xw);
            between();
            store_round(threadIdx.x, xw);
            __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0_only());
            piece_barrier();
        } else {
            for (int t0 = threadIdx.x; t0 < MT * PRP; t0 += XB * kPieceThreads) {
                uint32_t xw[XB][KW];
                load_round(t0, xw);
                store_round(t0, xw);
            }
            __syncthreads();
        }
    };
    auto load_x = [&](auto&& between, auto EarlyC) __attribute__((always_inline)) {
        constexpr int Early = decltype(EarlyC)::value;
        if constexpr (XREG && BITS == 0) {
            // dense operands are x itself: each lane loads its own
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
            stage_x(between, Int<Early>{});
            if constexpr (XREG) {
                // affine, registers: each lane copies its own operands
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const int p = li + P * j;
#pragma unroll
                        for (int c = 0; c < NCHP; ++c) {
                            const uint4 v = xp[(m * NCHP + c) * PRP + p];
                            xq[j][m][4 * c] = v.x; xq[j][m][4 * c + 1] = v.y;
                            xq[j][m][4 * c + 2] = v.z; xq[j][m][4 * c + 3] = v.w;
                        }
                        const float2 v = xc[m * PRP + p];
                        xX[j][m] = v.x;
                        xT[j][m] = v.y;
                    }
            }
        }
    };

    // ---- output staging: G*MT fp32 per finished tile, wavefront-private
    float* obuf = reinterpret_cast<float*>(
                      (XREG && BITS == 0) ? lds_p4
                           : lds_p4 + (size_t)MT * NCHP * PRP + (BITS != 0 ? ((size_t)MT * PRP + 1) / 2 : 0))
                  + (size_t)wave * a.tmax * PER_TILE;

    // ---- lane offsets within a tile (loop-invariant)
    // gsrc[j]: byte address (for ds_bpermute) of the lane holding piece j's
    // group (lane g holds the tile's group g); a lane slot past the row's end
    // points at some group of the tile, its x operands are zero
    uint32_t woff[J];
    [[maybe_unused]] int gsrc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int p = li + P * j;
        woff[j] = (uint32_t)(slot * row_bytes + (int64_t)p * 16);
        gsrc[j] = ((slot * gpr + p / PG::PPG) & 63) * 4;
    }

    // ---- ring of D = RD*J slots; slot d holds piece j = d % J of a row tile
    uint32_t wb[D][S][4];
    [[maybe_unused]] uint32_t sw[S][RD], bw[S][RD];   // per stream and ring row: the scale / bias of group `lane`
    int64_t f_tile = wg * CT;   // tile being fetched (wave-uniform)
    int f_c = 0;                // its index within the super-tile
    __amdgpu_buffer_rsrc_t rw[S], rs[S], rb[S];
    auto set_tile = [&]() __attribute__((always_inline)) {
        const void* w0 = a.w0;
        const uint16_t* sc0 = a.scales;
        const uint16_t* bi0 = a.biases;
        int64_t n0 = f_tile * G;
        int64_t nrows = a.N;
        if constexpr (SEG) {
            // the projection holding this tile: scalar selects, no branch
            const int sg = seg_of(a, n0);
            w0 = seg_pick(a.seg_w, sg);
            sc0 = seg_pick(a.seg_scales, sg);
            bi0 = seg_pick(a.seg_biases, sg);
            nrows = seg_rows(a, sg);
            n0 -= seg_start(a, sg);
        }
        // The descriptors cover this tile's rows that exist (0..G): every
        // load of a tile lies within its G rows (weights at woff, the G*K/64
        // <= 64 scales and biases at lane*2), so the range needs one clamp
        // per tile, not one per descriptor.
        const int rt = rows_in_tile(nrows - n0, G);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            rw[s] = make_rsrc(static_cast<const char*>(s == 0 ? w0 : a.w1) + n0 * row_bytes, rt * (int)row_bytes);
            if constexpr (BITS != 0) {
                rs[s] = make_rsrc((s == 0 ? sc0 : a.scales1) + n0 * gpr, rt * gpr * 2);
                rb[s] = make_rsrc((s == 0 ? bi0 : a.biases1) + n0 * gpr, rt * gpr * 2);
            }
        }
    };
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    auto fetch = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        constexpr int j = d % J;
        if constexpr (j == 0) {
            set_tile();
            // issued before the row's first piece, so waiting for that piece
            // covers them; consume(d) of the row's first piece has already
            // taken the previous values out (fetch(d) follows consume(d))
            if constexpr (BITS != 0) {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    sw[s][d / J] = __builtin_amdgcn_raw_buffer_load_b16(rs[s], (uint32_t)lane * 2, 0, kLoadNT);
                    bw[s][d / J] = __builtin_amdgcn_raw_buffer_load_b16(rb[s], (uint32_t)lane * 2, 0, kLoadNT);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw[s], woff[j], 0, kLoadNT);
            wb[d][s][0] = v.x; wb[d][s][1] = v.y; wb[d][s][2] = v.z; wb[d][s][3] = v.w;
        }
        if constexpr (j == J - 1) {
            ++f_tile;
            if (++f_c == CT) { f_c = 0; f_tile += (W - 1) * CT; }
        }
    };

    float acc[S][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[s][m] = 0.0f;
    int ti = 0;                 // tiles finished by this wavefront
    [[maybe_unused]] float rsc[S][J], rbi[S][J];   // scale and bias of each piece of the row in use, per stream

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        constexpr int j = d % J;
        const int p = li + P * j;
        // x in LDS is loop-invariant; the fence keeps its reads here instead
        // of letting them be hoisted out of the loop into registers
        if constexpr (!XREG) code_fence();
        if constexpr (BITS == 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint32_t xv[4];
                if constexpr (XREG) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[i] = xq[j][m][i];
                } else {
                    const uint4 v = xp[m * PRP + p];
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
            // (per weight stream: the fused SwiGLU runs its gate and up rows
            // through the same x operands)
            float dd[S][MT], de[S][MT];
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int m = 0; m < MT; ++m) dd[s][m] = de[s][m] = 0.0f;
            static_for<0, NCHP>([&](auto C) __attribute__((always_inline)) {
                constexpr int c = decltype(C)::value;
                uint32_t q[S][4];
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    q[s][0] = Plan::template pair<4 * c + 0>(wb[d][s]);
                    q[s][1] = Plan::template pair<4 * c + 1>(wb[d][s]);
                    q[s][2] = Plan::template pair<4 * c + 2>(wb[d][s]);
                    q[s][3] = Plan::template pair<4 * c + 3>(wb[d][s]);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    uint32_t x0, x1, x2, x3;
                    if constexpr (XREG) {
                        x0 = xq[j][m][4 * c]; x1 = xq[j][m][4 * c + 1];
                        x2 = xq[j][m][4 * c + 2]; x3 = xq[j][m][4 * c + 3];
                    } else {
                        const uint4 v = xp[(m * NCHP + c) * PRP + p];
                        x0 = v.x; x1 = v.y; x2 = v.z; x3 = v.w;
                    }
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        float v0 = dd[s][m], v1 = de[s][m];
                        v0 = dot2(q[s][0], x0, v0);
                        v1 = dot2(q[s][1], x1, v1);
                        v0 = dot2(q[s][2], x2, v0);
                        v1 = dot2(q[s][3], x3, v1);
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
            if constexpr (j == 0) {
                // the row's first piece takes every piece's scale and bias
                // (widened to fp32 once, in the lane that loaded them)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int sf = (int)(sw[s][d / J] << 16), bf = (int)(bw[s][d / J] << 16);
#pragma unroll
                    for (int jj = 0; jj < J; ++jj) {
                        rsc[s][jj] = __int_as_float(__builtin_amdgcn_ds_bpermute(gsrc[jj], sf));
                        rbi[s][jj] = __int_as_float(__builtin_amdgcn_ds_bpermute(gsrc[jj], bf));
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float X, Tc;
                if constexpr (XREG) {
                    X = xX[j][m];
                    Tc = xT[j][m];
                } else {
                    const float2 v = xc[m * PRP + p];
                    X = v.x;
                    Tc = v.y;
                }
#pragma unroll
                for (int s = 0; s < S; ++s)
                    acc[s][m] = fmaf(rsc[s][j], (dd[s][m] + de[s][m]) - Tc, fmaf(rbi[s][j], X, acc[s][m]));
            }
        }
        if constexpr (j == J - 1) {
            // end of a row tile: segment sums, epilogue, stage, reset.  Lane li
            // of a segment stages outputs m = li mod MT (+ P, + 2P, ... when
            // MT > P); lanes holding the same m write the same value.
            float out[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float v = segment_sum64_ct<L>(acc[0][m]);
                if constexpr (SWIGLU) {
                    const float u = segment_sum64_ct<L>(acc[1][m]);
                    v = (v / (1.0f + __expf(-v))) * u;
                }
                out[m] = v;
#pragma unroll
                for (int s = 0; s < S; ++s) acc[s][m] = 0.0f;
            }
            constexpr int NV = MT > P ? MT / P : 1;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int m0 = (li & (MT - 1) & (P - 1)) + v * P;
                float val = out[0];
#pragma unroll
                for (int m = 1; m < MT; ++m) val = (m == m0) ? out[m] : val;
                obuf[ti * PER_TILE + slot * MT + m0] = val;
            }
            ++ti;
        }
    };

    // prologue: RD rows, unconditionally (tiles past the wavefront's share --
    // all of them for a wavefront with no tiles -- read as zero or as valid
    // rows; they are never consumed), and x.  x is loaded first: dense x in
    // registers because the loop reads it, and a load issued after the
    // weights would make every wait in the loop a wait for all loads in
    // flight; staged operands of one round because their arithmetic then
    // waits for x only and overlaps the weights' latency (the weights go out
    // between the x loads and that arithmetic).
    auto fetch_ring = [&]() __attribute__((always_inline)) {
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(Dd); });
    };
    // (staged x of more than one round -- dense M = 8 with long rows, ~32 KB
    // per CU -- goes after the weights instead: loaded first it delayed the
    // weight stream, 7.5 -> 9.1 us on 1536 x 4096)
    constexpr bool XFIRST = (int64_t)MT * PRP <= (int64_t)(BITS == 0 ? 8 : 2) * kPieceThreads;
    if constexpr (XREG && BITS == 0) {
        load_x([]() {}, Int<0>{});
        fetch_ring();
    } else if constexpr (XFIRST) {
        load_x(fetch_ring, Int<1>{});
    } else {
        fetch_ring();
        load_x([]() {}, Int<0>{});
    }
    if (my_tiles == 0) {
        if (a.amx && lane < MT) amx_store(a.amx, a.amx_slots, wg, lane, amx_neutral_value(), kAmxNoIndex);
        return;
    }
    // 32-bit loop counts (a wavefront's tiles fit easily): a signed 64-bit
    // compare would run on the vector unit once per step
    const int nt = (int)my_tiles;
    int bt = 0;
    for (; bt + 2 * RD <= nt; bt += RD) {                // steady state
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            // raised priority from a slot's arithmetic through its next loads:
            // a wavefront whose data has arrived finishes with it and refills
            // its slot before the others take the SIMD (measured 2-5% faster
            // on the 4-bit LM head at M = 1)
            __builtin_amdgcn_s_setprio(2);
            consume(Dd);
            fetch(Dd);
            __builtin_amdgcn_s_setprio(0);
            // keep this order: without the barrier the scheduler sinks the
            // loads below the next slots' arithmetic, and each slot then waits
            // for every load in flight (vmcnt(0)) instead of its own
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    for (; bt < nt; bt += RD) {                         // drain
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int r = decltype(Dd)::value / J;
            if (bt + r < nt) {
                consume(Dd);
                if (bt + r + RD < nt) fetch(Dd);
            }
        });
    }

    // write out the staged outputs: value v of the wavefront's list is tile
    // v / (G*MT), row slot (v / MT) % G, output row m = v % MT
    if (a.amx) {
        // row argmax instead: lane l only sees outputs of row m = l % MT
        // (64 and G*MT are multiples of MT), so it keeps one running maximum;
        // the lanes of a row combine theirs and lane m writes the
        // wavefront's partial of row m
        float bv = amx_neutral_value();
        int bi = kAmxNoIndex;
        for (int v = lane; v < ti * PER_TILE; v += 64) {
            const int t2 = v / PER_TILE;
            const int r = v % PER_TILE;
            const int m = r % MT;
            const int64_t tile = (wg + (int64_t)(t2 / CT) * W) * CT + t2 % CT;
            const int64_t n = tile * G + r / MT;
            if (m < a.M && n < a.N) amx_take(bv, bi, obuf[v], (int)n);
        }
        if constexpr (MT == 1) {
            // one row: the DPP row tree, then the lane swaps across 16 and 32
            amx_row(bv, bi);
            amx_xor(bv, bi, 16);
            amx_xor(bv, bi, 32);
        } else {
#pragma unroll
            for (int sh = MT; sh < 64; sh <<= 1) amx_xor(bv, bi, sh);
        }
        if (lane < MT) amx_store(a.amx, a.amx_slots, wg, lane, bv, bi);
        return;
    }
    for (int v = lane; v < ti * PER_TILE; v += 64) {
        const int t2 = v / PER_TILE;
        const int r = v % PER_TILE;
        const int m = r % MT;
        const int64_t tile = (wg + (int64_t)(t2 / CT) * W) * CT + t2 % CT;
        const int64_t n = tile * G + r / MT;
        if (m < a.M && n < a.N) {
            const float val = obuf[v];
            void* y = a.y;
            int64_t nl = n, ny = a.N;
            if constexpr (SEG) {                 // the projection holding row n
                const int sg = seg_of(a, n);
                y = seg_pick(a.seg_y, sg);
                nl = n - seg_start(a, sg);
                ny = seg_rows(a, sg);
            }
            const size_t o = (size_t)m * ny + nl;
            if (a.out_f32) reinterpret_cast<float*>(y)[o] = val;
            else reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16_rne(val);
        }
    }
}

// LDS bytes of one workgroup: staged x operands (none for dense x in
// registers; affine operands are staged on the way to registers) plus the
// output staging for `tmax` tiles per wavefront.
template <int BITS>
size_t piece_lds_bytes(int MT, bool xreg, int L, int J, int K, int64_t tmax)
{
    (void)K;
    const int G = 64 >> L;
    const size_t out = (size_t)(kPieceThreads / 64) * tmax * G * MT * 4;
    if (xreg && BITS == 0) return out;       // dense x goes straight to registers
    const size_t PRP = (size_t)J << L;
    const size_t x16 = (size_t)MT * (PieceGeo<BITS>::NPP / 4) * PRP + (BITS != 0 ? ((size_t)MT * PRP + 1) / 2 : 0);
    return x16 * 16 + out;
}

template <int BITS, int MT, bool SW, bool XREG, int L, int J, bool SEG>
hipError_t launch_piece_one(const ProjArgs& a, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&piece_kernel<BITS, MT, SW, XREG, L, J, SEG>);
    {
        hipError_t e = raise_lds_limit(fn, kPieceLdsMax);
        if (e != hipSuccess) return e;
    }
    int cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    constexpr int64_t G = 64 >> L;
    constexpr int NW = kPieceThreads / 64;
    const int64_t T = ((int64_t)a.N + G - 1) / G;
    const int64_t row_bytes = BITS == 0 ? (int64_t)a.K * 2 : (int64_t)a.K * BITS / 8;
    // super-tiles of consecutive rows (sizes measured on the LM heads), but
    // no fewer super-tiles than wavefront slots (a small matrix is spread
    // over all CUs, not batched onto a few wavefronts)
    int64_t ct = (BITS == 0 ? 8192 : 4096) / (G * row_bytes);    // ~8 KB dense, ~4 KB affine
    if (ct < 1) ct = 1;
    {
        int bpc = 0;
        e = occupancy(bpc, fn, kPieceThreads, piece_lds_bytes<BITS>(MT, XREG, L, J, a.K, (T + (int64_t)cus * NW - 1) / ((int64_t)cus * NW) + ct));
        if (e != hipSuccess) return e;
        if (bpc < 1) bpc = 1;
        if (bpc * NW > piece_max_waves_per_cu<BITS, MT>()) bpc = piece_max_waves_per_cu<BITS, MT>() / NW;
        const int64_t slots = (int64_t)bpc * cus * NW;
        if (ct > 1 && T / ct < slots) ct = T / slots > 1 ? T / slots : 1;
    }
    const int64_t st = (T + ct - 1) / ct;
    // Grid: the wavefront slots the device holds at once at this LDS size, at
    // most piece_max_waves_per_cu per CU (the output staging depends on the
    // grid: settle in a few rounds).
    int64_t waves = st, tmax = 0;
    size_t lds = 0;
    for (int round = 0; round < 3; ++round) {
        tmax = ((st + waves - 1) / waves) * ct;
        lds = piece_lds_bytes<BITS>(MT, XREG, L, J, a.K, tmax);
        if (lds > kPieceLdsMax) return hipErrorInvalidValue;
        int bpc = 0;
        e = occupancy(bpc, fn, kPieceThreads, lds);
        if (e != hipSuccess) return e;
        if (bpc < 1) bpc = 1;
        if (bpc * NW > piece_max_waves_per_cu<BITS, MT>()) bpc = piece_max_waves_per_cu<BITS, MT>() / NW;
        int64_t w = (int64_t)bpc * cus * NW;
        if (w > st) w = st;
        if (w == waves && round > 0) break;
        waves = w;
    }
    const int blocks = (int)((waves + NW - 1) / NW);
    if (a.amx && (int64_t)blocks * NW > a.amx_slots) return hipErrorInvalidValue;   // one partial per wavefront
    if (a.amx_producers) *a.amx_producers = (int64_t)blocks * NW;
    // the kernel deals super-tiles over all blocks*NW wavefronts
    tmax = ((st + (int64_t)blocks * NW - 1) / ((int64_t)blocks * NW)) * ct;
    lds = piece_lds_bytes<BITS>(MT, XREG, L, J, a.K, tmax);
    if (lds > kPieceLdsMax) return hipErrorInvalidValue;
    ProjArgs a2 = a;
    a2.tpw = ct;
    a2.tmax = tmax;
    hipLaunchKernelGGL((piece_kernel<BITS, MT, SW, XREG, L, J, SEG>), dim3(blocks), dim3(kPieceThreads), lds, s, a2);
    return hipGetLastError();
}

template <int BITS, int MT, bool SW, int L, int J>
hipError_t launch_piece_mt(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    constexpr bool XR = piece_xreg_ok<BITS, MT, J>();
    if ((c.xreg != 0) != XR) return hipErrorInvalidValue;
    if constexpr (!SW) {
        if (a.nseg > 1) return launch_piece_one<BITS, MT, SW, XR, L, J, true>(a, s);
    }
    return launch_piece_one<BITS, MT, SW, XR, L, J, false>(a, s);
}

template <int BITS, bool SW, int L, int J>
hipError_t launch_piece_lj(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.MT) {
        case 1: return launch_piece_mt<BITS, 1, SW, L, J>(a, c, s);
        case 2: return launch_piece_mt<BITS, 2, SW, L, J>(a, c, s);
        case 4: return launch_piece_mt<BITS, 4, SW, L, J>(a, c, s);
        case 8: return launch_piece_mt<BITS, 8, SW, L, J>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

// The (2^L lanes per row, J pieces per lane) pairs the geometry choice uses.
template <int BITS, bool SW>
hipError_t launch_piece_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    switch (c.lpr_log2 * 16 + c.pieces_per_lane) {
        case 6 * 16 + 1: return launch_piece_lj<BITS, SW, 6, 1>(a, c, s);
        case 6 * 16 + 2: return launch_piece_lj<BITS, SW, 6, 2>(a, c, s);
        case 6 * 16 + 3: return launch_piece_lj<BITS, SW, 6, 3>(a, c, s);
        case 6 * 16 + 4: return launch_piece_lj<BITS, SW, 6, 4>(a, c, s);
        case 6 * 16 + 8: return launch_piece_lj<BITS, SW, 6, 8>(a, c, s);
        case 4 * 16 + 1: return launch_piece_lj<BITS, SW, 4, 1>(a, c, s);
        case 4 * 16 + 2: return launch_piece_lj<BITS, SW, 4, 2>(a, c, s);
        case 4 * 16 + 3: return launch_piece_lj<BITS, SW, 4, 3>(a, c, s);
        case 4 * 16 + 4: return launch_piece_lj<BITS, SW, 4, 4>(a, c, s);
        case 3 * 16 + 1: return launch_piece_lj<BITS, SW, 3, 1>(a, c, s);
        case 2 * 16 + 1: return launch_piece_lj<BITS, SW, 2, 1>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
