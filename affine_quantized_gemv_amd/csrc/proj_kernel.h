// Small-M projection kernels for gfx950 (CDNA4, wave64): VALU path.
//
// One template covers the dense bf16 GEMV, the affine b-bit GEMVs and the
// fused up/gate SwiGLU.  Data flow per workgroup:
//
//   1. Stage x (all M rows, one K-tile) into LDS.  Dense: as is.  Affine: in
//      the order and pre-scaling the width's pair plan needs (pair_plans.h),
//      plus two fp32 constants per (row m, group): X = sum of the group's x
//      and T = 128 * sum of its pre-scaled x.  The x loads are issued first,
//      then the first weight loads, so HBM latency overlaps the staging.
//   2. Each wavefront owns G*R weight rows.  Its 64 lanes form G segments of
//      2^L lanes; a segment streams one row, each lane taking every 2^L-th
//      "unit" of it (8 k = 16 bytes dense; one 64-code group = 8b bytes
//      affine), so every weight byte is read from HBM exactly once.  A ring
//      of D units per lane keeps D loads in flight while one is computed.
//   3. Dense: acc += dot2(W pair, x pair).  Affine: 32 (64 for b = 8) bf16x2
//      operands 0x43004300 | code fields are built from the packed words with
//      masks (no lookup tables), d = sum dot2(operand, pre-scaled x pair), then
//      acc += scale*(d - T) + bias*X, all in fp32 -- the group's algebraically
//      exact factored form of sum_k x*(scale*q + bias).
//   4. Segment sums (DPP within 16 lanes, lane shuffles across 16 and 32; one
//      fixed tree), then a fused epilogue: fp32 or RNE bf16 store; SwiGLU
//      applies silu(g)*u in fp32 first.
//
// Formats: AstrAI decode_linear_benchmark.md (commit message: BF16 decode
// GEMV, fused BF16 up/gate SwiGLU); TensorFold PR #849 "qwen3_5 cuda:
// mixed-width MLX checkpoints, 2 to 8 bits in groups of 64" (affine widths,
// groups of 64).  Mask-based code placement instead of lookups: FreeToken-Kai
// docs/turing.md, section 5.
#pragma once
#include "aqg_device.h"
#include "host_query.h"
#include "kernels.h"
#include "pair_plans.h"

namespace aqg {
namespace detail {

constexpr int kMaxThreads = 256;
constexpr size_t kLdsBudget = 64 * 1024;

template <int BITS> struct Geo {
    static constexpr int UK = 64;             // k per unit (one group)
    static constexpr int NW = 2 * BITS;       // uint32 words per unit
    static constexpr int NP = PairPlan<BITS>::NP;
    static constexpr int NCH = NP / 4;        // uint4 x-chunks per (m, unit)
    static constexpr int LDS_PER_UNIT = 16 * NCH + 8;  // bytes per (m, unit)
    static constexpr int D = 2;               // units in flight per lane
};
template <> struct Geo<0> {
    static constexpr int UK = 8;
    static constexpr int NW = 4;
    static constexpr int NP = 4;
    static constexpr int NCH = 1;
    static constexpr int LDS_PER_UNIT = 16;
    static constexpr int D = 4;
};

__device__ __forceinline__ uint32_t half_of(const uint32_t* xw, int k)
{
    return (xw[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

// Load one unit (NW words) of a row.  Even widths and dense: 16-byte loads;
// odd widths: 8-byte loads (a group of an odd width is 8b bytes).  Weights are
// read once, so the loads are non-temporal.
template <int BITS>
__device__ __forceinline__ void load_unit(const uint32_t* __restrict__ p, uint32_t* w)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int NW = Geo<BITS>::NW;
    if constexpr (NW % 4 == 0) {
        const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            u32x4 v = __builtin_nontemporal_load(q + i);
            w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else {
        const u32x2* q = reinterpret_cast<const u32x2*>(p);
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) {
            u32x2 v = __builtin_nontemporal_load(q + i);
            w[2 * i + 0] = v.x; w[2 * i + 1] = v.y;
        }
    }
}

// ---------------------------------------------------------------- staging

// Pre-scaled pair operands and constants of the x values that one plan covers
// (a 64-k group for PairPlan, a 16-byte piece's 128/b k for PiecePlan), in the
// plan's order: xq[i] = (x[LO_K] * 2^LO_E) | (x[HI_K] * 2^HI_E) << 16,
// X = sum of the covered x (each code once: its significance-0 subcode), and
// T = the code offset 128 * (sum of the pre-scaled halves) as the consumers'
// own chain computes it: the same v_dot2 sequence over the same operands
// (pairs 4c, 4c + 2 into one sum, 4c + 1, 4c + 3 into the other, then their
// sum) with every code field zero, i.e. the pair 0x43004300 = (128, 128).
// A unit whose codes are all zero therefore gives d == T bit for bit and
// contributes exactly bias * X, not a rounding residue of the offset; other
// codes leave the usual fp32 rounding of d.  Every caller uses this one
// routine, so the constants are identical wherever x is kept.
template <class P, int NXW>
__device__ __forceinline__ void plan_x_operands(const uint32_t (&xw)[NXW], uint32_t (&xq)[P::NP],
                                                float& X, float& T)
{
    static_assert(P::NP % 4 == 0, "the consumers take pairs four at a time");
    float xs = 0.0f;
    static_for<0, P::NP>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const uint32_t hl = half_of(xw, P::LO_K[i]);
        const uint32_t hh = half_of(xw, P::HI_K[i]);
        if constexpr (P::LO_E[i] + P::LO_P[i] == 0) xs += bf16_to_f32(hl);
        if constexpr (P::HI_E[i] + P::HI_P[i] == 0) xs += bf16_to_f32(hh);
        const uint32_t lo = bf16_scale_pow2<P::LO_E[i]>(hl);
        const uint32_t hi = bf16_scale_pow2<P::HI_E[i]>(hh);
        xq[i] = lo | (hi << 16);
    });
    float t0 = 0.0f, t1 = 0.0f;
    static_for<0, P::NP / 4>([&](auto C) __attribute__((always_inline)) {
        constexpr int c = decltype(C)::value;
        t0 = dot2(kZeroCodePair, xq[4 * c + 0], t0);
        t1 = dot2(kZeroCodePair, xq[4 * c + 1], t1);
        t0 = dot2(kZeroCodePair, xq[4 * c + 2], t0);
        t1 = dot2(kZeroCodePair, xq[4 * c + 3], t1);
    });
    X = xs;
    T = t0 + t1;
}

template <int BITS>
__device__ __forceinline__ void group_x_operands(const uint32_t (&xw)[32], uint32_t (&xq)[PairPlan<BITS>::NP],
                                                 float& X, float& T)
{
    plan_x_operands<PairPlan<BITS>, 32>(xw, xq, X, T);
}

// A staging task is split into load (global -> registers) and store (compute
// and write LDS) so the caller can issue weight loads in between.

template <int BITS, int MT> struct Stager;

// Dense: task t = (m, u) copies 8 bf16: x[m][kt + 8u ..] -> xs[m*upm + u].
template <int MT> struct Stager<0, MT> {
    struct Regs { uint4 v; };
    const ProjArgs& a;
    int kt, upm;
    uint4* xs;
    __device__ int ntasks() const { return MT * upm; }
    __device__ Regs load(int t) const
    {
        const int m = t / upm, u = t - m * upm;
        Regs r;
        r.v = make_uint4(0, 0, 0, 0);
        if (m < a.M) r.v = *reinterpret_cast<const uint4*>(a.x + (size_t)m * a.K + kt + 8 * u);
        return r;
    }
    __device__ void store(int t, const Regs& r) const { xs[t] = r.v; }
};

// Affine: task t = (m, group g of the tile) writes NCH uint4 of pre-scaled bf16
// pairs in plan order to xp[(m*NCH + c)*ngt + g] and (X, T) to xc[m*ngt + g].
template <int BITS, int MT> struct Stager {
    struct Regs { uint32_t xw[32]; };
    const ProjArgs& a;
    int kt, ngt;
    uint4* xp;
    float2* xc;
    __device__ int ntasks() const { return MT * ngt; }
    __device__ Regs load(int t) const
    {
        const int m = t / ngt, g = t - m * ngt;
        Regs r;
        if (m < a.M) {
            const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)m * a.K + kt + 64 * g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint4 v = src[i];
                r.xw[4 * i] = v.x; r.xw[4 * i + 1] = v.y; r.xw[4 * i + 2] = v.z; r.xw[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) r.xw[i] = 0;
        }
        return r;
    }
    __device__ void store(int t, const Regs& r) const
    {
        constexpr int NCH = Geo<BITS>::NCH;
        const int m = t / ngt, g = t - m * ngt;
        uint32_t xq[PairPlan<BITS>::NP];
        float X, T;
        group_x_operands<BITS>(r.xw, xq, X, T);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            xp[(m * NCH + c) * ngt + g] = make_uint4(xq[4 * c], xq[4 * c + 1], xq[4 * c + 2], xq[4 * c + 3]);
        xc[m * ngt + g] = make_float2(X, T);
    }
};

// Sum over aligned segments of 2^L lanes (L <= 6); every lane of a segment
// ends with the same bits.  Within 16 lanes: segment_sum's DPP tree; across
// 16 and 32: lane swaps adding two equal-shaped partial sums.
__device__ __forceinline__ float segment_sum64(float v, int L)
{
    v = segment_sum(v, L < 4 ? L : 4);
    if (L >= 5) v += __shfl_xor(v, 16);
    if (L >= 6) v += __shfl_xor(v, 32);
    return v;
}

// The same tree with the segment width fixed at compile time (no branches).
template <int L>
__device__ __forceinline__ float segment_sum64_ct(float v)
{
    if constexpr (L >= 1) v += dpp_f32<0xB1>(v);
    if constexpr (L >= 2) v += dpp_f32<0x4E>(v);
    if constexpr (L >= 3) v += dpp_f32<0x141>(v);
    if constexpr (L >= 4) v += dpp_f32<0x140>(v);
    if constexpr (L >= 5) v += __shfl_xor(v, 16);
    if constexpr (L >= 6) v += __shfl_xor(v, 32);
    return v;
}

// ------------------------------------------------------- per-unit arithmetic

// One unit of R rows (S weight streams, each with its own scales and
// biases) against x from LDS:
//   dense:  acc[s][r][m] += sum of 8 products (4 dot2)
//   affine: d = sum over the group's pairs of dot2(operand, x' pair);
//           acc += scale*(d - T) + bias*X.
// xp/xc: the tile's staged x (ut units per m row); u: unit within the tile.
template <int BITS, int MT, int S, int R>
__device__ __forceinline__ void unit_mac(const uint32_t (&w)[S][R][Geo<BITS>::NW], const float (&sc)[S][R],
                                         const float (&bi)[S][R], const uint4* xp, const float2* xc, int ut,
                                         int u, float (&acc)[S][R][MT])
{
    if constexpr (BITS == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xv = xp[m * ut + u];
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float v = acc[s][r][m];
                    v = dot2(w[s][r][0], xv.x, v);
                    v = dot2(w[s][r][1], xv.y, v);
                    v = dot2(w[s][r][2], xv.z, v);
                    v = dot2(w[s][r][3], xv.w, v);
                    acc[s][r][m] = v;
                }
        }
    } else {
        using P = PairPlan<BITS>;
        constexpr int NCH = Geo<BITS>::NCH;
        // two accumulators per output (even and odd pairs of each chunk), so
        // consecutive dot2 do not wait on each other; d = d0 + d1
        float dd[S][R][MT], de[S][R][MT];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) dd[s][r][m] = de[s][r][m] = 0.0f;
        static_for<0, NCH>([&](auto C) __attribute__((always_inline)) {
            constexpr int c = decltype(C)::value;
            uint32_t p[S][R][4];
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    p[s][r][0] = P::template pair<4 * c + 0>(w[s][r]);
                    p[s][r][1] = P::template pair<4 * c + 1>(w[s][r]);
                    p[s][r][2] = P::template pair<4 * c + 2>(w[s][r]);
                    p[s][r][3] = P::template pair<4 * c + 3>(w[s][r]);
                }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4 xv = xp[(m * NCH + c) * ut + u];
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float v0 = dd[s][r][m], v1 = de[s][r][m];
                        v0 = dot2(p[s][r][0], xv.x, v0);
                        v1 = dot2(p[s][r][1], xv.y, v1);
                        v0 = dot2(p[s][r][2], xv.z, v0);
                        v1 = dot2(p[s][r][3], xv.w, v1);
                        dd[s][r][m] = v0;
                        de[s][r][m] = v1;
                    }
            }
            // keep each chunk's operands and x reads local to it
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MT; ++m) { pin(dd[s][r][m]); pin(de[s][r][m]); }
            code_fence();
        });
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float2 xcv = xc[m * ut + u];
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[s][r][m] = fmaf(sc[s][r], (dd[s][r][m] + de[s][r][m]) - xcv.y, fmaf(bi[s][r], xcv.x, acc[s][r][m]));
        }
    }
}

// ----------------------------------------------------------------- kernel

template <int BITS, int MT, int R, bool SWIGLU>
__global__ void __launch_bounds__(kMaxThreads) proj_kernel(ProjArgs a)
{
    extern __shared__ uint4 lds_u4[];
    constexpr int S = SWIGLU ? 2 : 1;
    constexpr int UK = Geo<BITS>::UK;
    constexpr int NW = Geo<BITS>::NW;
    constexpr int NCH = Geo<BITS>::NCH;
    constexpr int D = Geo<BITS>::D;

    const int L = a.lpr_log2;
    const int LPR = 1 << L;
    const int G = 64 >> L;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane >> L;
    const int li = lane & (LPR - 1);
    const int nwaves = blockDim.x >> 6;

    const int64_t row0 = ((int64_t)blockIdx.x * nwaves + wave) * (int64_t)(G * R) + slot;
    int64_t nrow[R];
    const uint32_t* wrow[S][R];
    const uint16_t* srow[S][R];
    const uint16_t* brow[S][R];
    const int64_t row_words = (BITS == 0) ? (int64_t)a.K / 2 : (int64_t)a.K * BITS / 32;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        nrow[r] = row0 + (int64_t)r * G;
        const int64_t n = nrow[r] < a.N ? nrow[r] : (int64_t)a.N - 1;  // clamp: load, never store
        wrow[0][r] = reinterpret_cast<const uint32_t*>(a.w0) + n * row_words;
        if constexpr (SWIGLU) wrow[1][r] = reinterpret_cast<const uint32_t*>(a.w1) + n * row_words;
        if constexpr (BITS != 0) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                srow[s][r] = (s == 0 ? a.scales : a.scales1) + n * (a.K / 64);
                brow[s][r] = (s == 0 ? a.biases : a.biases1) + n * (a.K / 64);
            }
        }
    }

    float acc[S][R][MT];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[s][r][m] = 0.0f;

    // Ring of D units of weights (and their scale/bias) per lane.
    uint32_t wb[D][S][R][NW];
    float sb[D][S][R], bb[D][S][R];

    for (int kt = 0; kt < a.K; kt += a.KT) {
        const int kw = min(a.KT, a.K - kt);
        const int ut = kw / UK;            // units in this tile (a multiple of LPR)
        const int upl = ut >> L;           // units per lane in this tile
        const int ubase = kt / UK;         // unit index of the tile start within a row
        uint4* xp = lds_u4;
        float2* xc = reinterpret_cast<float2*>(lds_u4 + MT * NCH * ut);

        auto fetch = [&](int d, int u) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    load_unit<BITS>(wrow[s][r] + (int64_t)(ubase + u) * NW, wb[d][s][r]);
            if constexpr (BITS != 0) {
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        sb[d][s][r] = bf16_to_f32(srow[s][r][ubase + u]);
                        bb[d][s][r] = bf16_to_f32(brow[s][r][ubase + u]);
                    }
            }
        };

        // x loads for this thread's first staging task, then the first D
        // units of weights, then the staging arithmetic and LDS writes.
        using St = Stager<BITS, MT>;
        St st = [&] {
            if constexpr (BITS == 0) return St{a, kt, kw / 8, xp};
            else return St{a, kt, kw / 64, xp, xc};
        }();
        // Dense tasks are 16-byte copies: XB of them are loaded at once.
        constexpr int XB = (BITS == 0) ? 8 : 1;
        const int ntask = st.ntasks();
        const int nthr = blockDim.x;
        typename St::Regs xr[XB];
#pragma unroll
        for (int i = 0; i < XB; ++i)
            if ((int)threadIdx.x + i * nthr < ntask) xr[i] = st.load(threadIdx.x + i * nthr);
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int d = decltype(Dd)::value;
            if (d < upl) fetch(d, li + d * LPR);
        });
        if (kt > 0) __syncthreads();       // previous tile's x fully consumed
        for (int t0 = threadIdx.x; t0 < ntask; t0 += XB * nthr) {
            if (t0 != (int)threadIdx.x) {
#pragma unroll
                for (int i = 0; i < XB; ++i)
                    if (t0 + i * nthr < ntask) xr[i] = st.load(t0 + i * nthr);
            }
#pragma unroll
            for (int i = 0; i < XB; ++i)
                if (t0 + i * nthr < ntask) st.store(t0 + i * nthr, xr[i]);
        }
        __syncthreads();

        for (int base = 0; base < upl; base += D) {
            static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
                constexpr int d = decltype(Dd)::value;
                const int j = base + d;
                if (j < upl) {
                    const int u = li + j * LPR;
                    unit_mac<BITS, MT, S, R>(wb[d], sb[d], bb[d], xp, xc, ut, u, acc);
                    if (j + D < upl) fetch(d, u + D * LPR);
                }
                code_fence();
            });
        }
    }

    // Segment reduction and epilogue.
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[s][r][m] = segment_sum64(acc[s][r][m], L);

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool row_ok = nrow[r] < a.N;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float v = acc[0][r][m];
            if constexpr (SWIGLU) {
                const float g = v;
                v = (g / (1.0f + __expf(-g))) * acc[1][r][m];
            }
            const int idx = r * MT + m;
            if (row_ok && m < a.M && (idx & (LPR - 1)) == li) {
                const size_t o = (size_t)m * a.N + nrow[r];
                if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = v;
                else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(v);
            }
        }
    }
}

// One thread per 64-code group: unpack through the same pair plan the GEMV
// uses, and write the codes as bytes.
template <int BITS>
__global__ void __launch_bounds__(256) unpack_kernel(const uint32_t* __restrict__ Wq,
                                                     uint8_t* __restrict__ codes, int64_t ngroups)
{
    using P = PairPlan<BITS>;
    constexpr int NW = 2 * BITS;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ngroups) return;
    uint32_t w[NW];
    load_unit<BITS>(Wq + t * NW, w);
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0;
    constexpr uint32_t FM = (1u << P::SW) - 1u;
    static_for<0, P::NP>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const uint32_t p = P::template pair<i>(w);
        const uint32_t lo = (p >> P::LO_P[i]) & FM;
        const uint32_t hi = (p >> (16 + P::HI_P[i])) & FM;
        constexpr int klo = P::LO_K[i], khi = P::HI_K[i];
        constexpr int glo = P::LO_E[i] + P::LO_P[i], ghi = P::HI_E[i] + P::HI_P[i];  // significance
        c[klo >> 2] |= (lo << glo) << (8 * (klo & 3));
        c[khi >> 2] |= (hi << ghi) << (8 * (khi & 3));
    });
    uint4* dst = reinterpret_cast<uint4*>(codes + t * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
}

template <int BITS, int MT, int R, bool SW>
hipError_t launch_one(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    hipLaunchKernelGGL((proj_kernel<BITS, MT, R, SW>), dim3(c.blocks), dim3(64 * c.nwaves), c.lds, s, a);
    return hipGetLastError();
}

template <int BITS, bool SW>
hipError_t launch_bits_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
#define AQG_CASE_MT(MTV)                                                    \
    case MTV:                                                               \
        return c.R == 2 ? launch_one<BITS, MTV, 2, SW>(a, c, s)             \
                        : launch_one<BITS, MTV, 1, SW>(a, c, s);
    switch (c.MT) {
        AQG_CASE_MT(1)
        AQG_CASE_MT(2)
        AQG_CASE_MT(4)
        AQG_CASE_MT(8)
        AQG_CASE_MT(16)
        AQG_CASE_MT(32)
        default: return hipErrorInvalidValue;
    }
#undef AQG_CASE_MT
}

}  // namespace detail
}  // namespace aqg
