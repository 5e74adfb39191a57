// Multi-tile matrix-core kernel for affine GEMVs with 2- to 8-bit codes at
// K = 4096 and M = 1..16 (M = 17..32: one launch per 16-column half) on
// gfx950.
//
// Each workgroup takes at most NT = 1, 2 or 4 row tiles of 16 rows (XCD-
// aware order; the grid is at least ceil(tiles / NT)); its 8 wavefronts split
// each row's 64 groups, 8 per wavefront.  A wavefront loads its part of a
// tile straight into the lanes of the MFMA A operand, as the one-tile-per-
// workgroup kernel (affine_split.h) does: 2, 4 and 8 bits as whole-line loads
// of 128-byte k-blocks (rows 0..7 and 8..15, the row_ror:8 DPP select and the
// 4 x 4 lane-row transpose), 3, 5, 6, 7 bits as the words of each lane's
// 16-code window.  The scales and biases of the wavefront's groups come as
// one dword per lane (row r, groups 2c, 2c + 1).
//
// All loads of a workgroup go out at once, before any wait: x (range-checked
// buffer loads; padding columns r >= M read zeros without a memory access),
// then every tile's codes, scales and biases into registers, indexed with
// constants only.  The code is straight-line (no loop-carried loads), so the
// compiler's own wait counts stay exact, one tile per wait; a scheduling
// barrier keeps the x arithmetic after the tile loads.  Nothing goes through
// LDS copies, whose issue rate (about 1 KB per 100-190 cycles per CU) caps a
// copy-fed kernel near half the HBM rate.  Slots past a workgroup's last tile
// and rows past N read as zeros (range-checked buffer offsets).
//
// Arithmetic per group: two MFMA k-steps on the codes placed as bf16
// (128 + q; 8-bit codes as two nibble chains, the high one weighted 16) give
// D = sum_k (C + q_k) x_k; the lane adds scale * (D - D0) in fp32 (D0, the
// same chain on zero codes, so zero codes add exactly zero).  The bias terms
// sum_g bias_g X_g of the tile are one more MFMA: A holds the row's biases of
// groups 2c, 2c + 1 in three k-slots each, B the exact three-piece bf16
// split of X_g (hi, mid, lo) for the lane's column, so every product is
// exact and a zero bias adds exactly zero.  The wavefronts' partial 16 x 16
// tiles are summed through LDS in wavefront order (double-buffered: one
// barrier per tile), so results are deterministic and the same for every
// M <= 16.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).  Shapes: 4096-
// wide layers (4096 x 4096, 14336 x 4096) at decode batch sizes.
#pragma once
#include "affine_split.h"

namespace aqg {
namespace detail {

template <int BITS, int GW> struct BurstGeo {
    static constexpr bool NAT = affine_split_natural<BITS>();
    static constexpr int NWN = AffineTileWidth<BITS>::NWN;
    static constexpr int KPW = NAT ? 1 : GW * BITS / 16;            // 128-byte k-blocks per wavefront
    static constexpr int GPK = NAT ? 1 : AffineMma<NAT ? 4 : BITS>::GPK;
    static constexpr int NCW = NAT ? GW * NWN : KPW * 8;            // code dwords per lane per tile
    static constexpr int SPL = GW <= 8 ? 1 : GW / 8;                // scale dwords per lane per tile
    static_assert(GW % 2 == 0, "groups come in pairs");
    static_assert(NAT || (GW * BITS) % 16 == 0, "whole k-blocks per wavefront");
};

template <int BITS, int GW> struct BurstStage {
    uint32_t cw[BurstGeo<BITS, GW>::NCW];
    uint32_t sw[BurstGeo<BITS, GW>::SPL];
    uint32_t bw[BurstGeo<BITS, GW>::SPL];
};

// LDS: two partial areas [NWV][4][65] floats, then per wavefront its scale
// table [GW][16] floats.
template <int GW, int NWV> struct BurstLds {
    static constexpr int PART = NWV * 4 * 65;                        // floats per partial area
    static constexpr int TAB = GW * 16;                             // floats per wavefront
    static constexpr size_t BYTES = (size_t)(2 * PART + NWV * TAB) * 4;
};

// Raw x words of one group for lane quarter c (two 16-byte vectors), in the
// positions the width's A operands need:
//   3, 5, 6, 7 bits: x[16c .. 16c + 7], x[16c + 8 .. 16c + 15] (natural order);
//   2 bits: the same 16 values (k-step t uses x[16c + 4t + {0..3}] and
//           x[16c + 8 + 4t + {0..3}]);
//   4 bits: x[8c .. 8c + 7], x[32 + 8c .. 32 + 8c + 7] (k-step t: the t-th);
//   8 bits: k-step t's x[32t + 4c + {0..3}] and x[32t + 16 + 4c + {0..3}].
struct BurstX { uint4 v[2]; };

// rx covers the M rows of x, so a padding column's row (r >= M) is out of
// range and reads zeros; voff = the lane's row offset (bytes), soff = the
// group's offset within the row.
template <int BITS>
__device__ __forceinline__ BurstX burst_x_load(__amdgpu_buffer_rsrc_t rx, uint32_t voff, uint32_t soff, int c)
{
    BurstX o;
    auto b128 = [&](int e) __attribute__((always_inline)) {   // 8 values from element e of the group
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + 2 * e, soff, 0));
    };
    if constexpr (BITS == 4) {
        o.v[0] = b128(8 * c);
        o.v[1] = b128(32 + 8 * c);
    } else if constexpr (BITS == 8) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x2v_t p = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(rx, voff + 2 * (32 * t + 4 * c), soff, 0));
            const u32x2v_t q = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(rx, voff + 2 * (32 * t + 4 * c + 16), soff, 0));
            o.v[t] = make_uint4(p[0], p[1], q[0], q[1]);
        }
    } else {
        o.v[0] = b128(16 * c);
        o.v[1] = b128(16 * c + 8);
    }
    return o;
}

// x^T operand of k-step t of the group (t = 0, 1) in the k order of the
// width's A operands (as stage_x_operand / stage_x_natural place them), and
// the sum of its 8 values.
template <int BITS>
__device__ __forceinline__ u32x4_t burst_x_operand(const BurstX& x, int t, float& sum)
{
    uint32_t o[4];
    if constexpr (!(BITS == 2 || BITS == 4 || BITS == 8)) {
        const uint4 v = x.v[t];
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (BITS == 4) {
        // x at 32t + 8c + {0,4,1,5,2,6,3,7}
        const uint4 v = x.v[t];
        o[0] = (v.x & 0xFFFFu) | (v.z << 16); o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        o[2] = (v.y & 0xFFFFu) | (v.w << 16); o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
    } else if constexpr (BITS == 2) {
        // x at 16c + 4t + {0,8,1,9,2,10,3,11}
        const uint32_t px = t ? x.v[0].z : x.v[0].x, py = t ? x.v[0].w : x.v[0].y;
        const uint32_t qx = t ? x.v[1].z : x.v[1].x, qy = t ? x.v[1].w : x.v[1].y;
        o[0] = (px & 0xFFFFu) | (qx << 16); o[1] = (px >> 16) | (qx & 0xFFFF0000u);
        o[2] = (py & 0xFFFFu) | (qy << 16); o[3] = (py >> 16) | (qy & 0xFFFF0000u);
    } else {
        // x at 32t + 4c + {0,2,1,3, 16,18,17,19}
        const uint4 v = x.v[t];
        o[0] = (v.x & 0xFFFFu) | (v.y << 16); o[1] = (v.x >> 16) | (v.y & 0xFFFF0000u);
        o[2] = (v.z & 0xFFFFu) | (v.w << 16); o[3] = (v.z >> 16) | (v.w & 0xFFFF0000u);
    }
    sum = ((bf16_to_f32(o[0] & 0xFFFFu) + bf16_to_f32(o[0] >> 16)) + (bf16_to_f32(o[1] & 0xFFFFu) + bf16_to_f32(o[1] >> 16))) +
          ((bf16_to_f32(o[2] & 0xFFFFu) + bf16_to_f32(o[2] >> 16)) + (bf16_to_f32(o[3] & 0xFFFFu) + bf16_to_f32(o[3] >> 16)));
    return u32x4_t{o[0], o[1], o[2], o[3]};
}

// B operand of a 16 x 16 x 32 MFMA carrying two fp32 values u, v (groups
// 2c, 2c + 1 of the lane's quarter) as three bf16 pieces each, in k-slots
// 8c .. 8c + 5 (the last two zero): truncating to bf16 twice leaves a
// remainder of at most 8 significant bits, so u = hi + mid + lo exactly.
__device__ __forceinline__ u32x4_t burst_pieces(float u, float v)
{
    auto split = [](float f, uint32_t& h, uint32_t& m, uint32_t& l) __attribute__((always_inline)) {
        const uint32_t hb = __float_as_uint(f) & 0xFFFF0000u;
        const float rem = f - __uint_as_float(hb);
        const uint32_t mb = __float_as_uint(rem) & 0xFFFF0000u;
        const float lo = rem - __uint_as_float(mb);
        h = hb >> 16; m = mb >> 16; l = __float_as_uint(lo) >> 16;
    };
    uint32_t uh, um, ul, vh, vm, vl;
    split(u, uh, um, ul);
    split(v, vh, vm, vl);
    return u32x4_t{uh | (um << 16), ul | (vh << 16), vm | (vl << 16), 0u};
}

template <int BITS, int GW, int NWV, int NT>
__global__ void __launch_bounds__(64 * NWV) affine_burst_kernel(ProjArgs a)
{
    using G = BurstGeo<BITS, GW>;
    using L = BurstLds<GW, NWV>;
    constexpr bool NAT = G::NAT;
    constexpr int K = 64 * GW * NWV;
    constexpr int ROWB = K * BITS / 8;
    constexpr int GPR = K / 64;
    constexpr int NWN = G::NWN;
    extern __shared__ float burst_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;
    const int r = lane & 15;
    const int g0 = wave * GW;                                       // first group of this wavefront

    const int64_t T = ((int64_t)a.N + 15) / 16;
    const int64_t G8 = gridDim.x / 8;
    const int64_t first = (gridDim.x % 8 == 0) ? (int64_t)(blockIdx.x % 8) * G8 + blockIdx.x / 8 : blockIdx.x;
    const int64_t stride = gridDim.x;
    const int64_t ntile = first < T ? (T - first + stride - 1) / stride : 0;

    // whole-matrix descriptors: a row past N (in a partial last tile) is out
    // of range and reads as zero
    const __amdgpu_buffer_rsrc_t rw = tile_rsrc(a.w0, (int64_t)a.N * ROWB);
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.scales, (int64_t)a.N * GPR * 2);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc(a.biases, (int64_t)a.N * GPR * 2);
    const uint32_t voff = NAT ? (uint32_t)(r * ROWB + 4 * ((16 * BITS * c) >> 5))
                              : (uint32_t)((r & 7) * ROWB + 16 * ((r < 8 ? 0 : 4) + c));
    // scales: lane (pair p, row) takes groups g0 + 2p, g0 + 2p + 1 of its row
    // (pairs past the wavefront's repeat the first ones)
    uint32_t soff[G::SPL];
#pragma unroll
    for (int q = 0; q < G::SPL; ++q) {
        const int p = ((lane >> 4) + 4 * q) % (GW / 2);
        soff[q] = (uint32_t)((r * GPR + g0 + 2 * p) * 2);
    }

    auto load = [&](int64_t j, BurstStage<BITS, GW>& st) __attribute__((always_inline)) {
        const int64_t t0 = first + j * stride;
        const int64_t t = t0 < T ? t0 : T;   // past the end: offsets out of range, zeros
        const uint32_t vw = voff + (uint32_t)(t * 16 * ROWB);
        if constexpr (NAT) {
#pragma unroll
            for (int g = 0; g < GW; ++g)
#pragma unroll
                for (int q = 0; q < NWN; ++q)
                    st.cw[g * NWN + q] = __builtin_amdgcn_raw_buffer_load_b32(rw, vw + 4 * q, (g0 + g) * 8 * BITS, kLoadNT);
        } else {
#pragma unroll
            for (int p = 0; p < G::KPW; ++p) {
                const int koff = 128 * (wave * G::KPW + p);
                // rows 8..15 through the vector offset (the range-checked part)
                const u32x4_t lo = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, vw, koff, kLoadNT));
                const u32x4_t hi = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, vw + 8 * ROWB, koff, kLoadNT));
#pragma unroll
                for (int i = 0; i < 4; ++i) { st.cw[8 * p + i] = lo[i]; st.cw[8 * p + 4 + i] = hi[i]; }
            }
        }
        const uint32_t vs = (uint32_t)(t * 16 * GPR * 2);
#pragma unroll
        for (int q = 0; q < G::SPL; ++q) {
            st.sw[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs + soff[q], 0, kLoadNT);
            st.bw[q] = __builtin_amdgcn_raw_buffer_load_b32(rb, vs + soff[q], 0, kLoadNT);
        }
    };

    // x (raw words only; padding columns r >= M read zeros); the operands
    // are composed below
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(a.x, (int64_t)a.M * K * 2);
    const uint32_t xvoff = (uint32_t)((r * K + 64 * g0) * 2);
    BurstX xr[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) xr[g] = burst_x_load<BITS>(rx, xvoff, (uint32_t)(128 * g), c);
    // all of the workgroup's tiles go out at once (straight-line code: the
    // compiler's wait counts stay exact, one tile per wait); slots past the
    // workgroup's last tile read zeros
    BurstStage<BITS, GW> slot[NT];
    static_for<0, NT>([&](auto Uc) __attribute__((always_inline)) {
        constexpr int u = decltype(Uc)::value;
        load(u, slot[u]);
    });
    // nothing moves across: the weight loads must be issued before the x
    // arithmetic below waits for x
    __builtin_amdgcn_sched_barrier(0);

    // x^T operands of the wavefront's 2 GW k-steps, group sums over the four
    // lane quarters (fixed order) and code offsets
    static_assert(GW == 8, "the pieces operands carry 2 groups per lane quarter");
    u32x4_t xb[2 * GW];
    float X[GW], z0[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
        float s0 = 0.f, s1 = 0.f;
        xb[2 * g] = burst_x_operand<BITS>(xr[g], 0, s0);
        xb[2 * g + 1] = burst_x_operand<BITS>(xr[g], 1, s1);
        const float v = s0 + s1;
        const float v16 = __shfl_xor(v, 16);
        const float p = (c & 1) ? v16 + v : v + v16;
        const float p32 = __shfl_xor(p, 32);
        X[g] = (c & 2) ? p32 + p : p + p32;
        const u32x4_t Z = u32x4_t{kZeroCodePair, kZeroCodePair, kZeroCodePair, kZeroCodePair};
        f32x4_t d0 = mfma16x16x32(Z, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
        d0 = mfma16x16x32(Z, xb[2 * g + 1], d0);
        // column r's offset sits in every row of the lane's accumulator
        z0[g] = BITS == 8 ? fmaf(16.0f, d0[0], d0[0]) : d0[0];   // 8 bits: the high-nibble chain is the same
    }
    // per tile, sum_g bias X_g is one MFMA: A = the row's biases of groups
    // 2c, 2c + 1, three slots each, B = the pieces of X of those groups for
    // the lane's column (products exact; a zero bias adds exactly zero)
    float xs0 = X[0], xs1 = X[1];
#pragma unroll
    for (int q = 1; q < GW / 2; ++q) {
        xs0 = c == q ? X[2 * q] : xs0;
        xs1 = c == q ? X[2 * q + 1] : xs1;
    }
    const u32x4_t bx = burst_pieces(xs0, xs1);

    uint32_t cmask = NAT ? AffineTileWidth<BITS>::MASK : AffineMma<NAT ? 4 : BITS>::MASK, cbias = kZeroCodePair;
    uint32_t cmaskh = AffineTileWidth<BITS>::MASK << 16;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+s"(cmaskh));
    asm volatile("" : "+v"(cbias));
    const uint32_t wsh = (uint32_t)((16 * BITS * c) & 31);   // odd widths: 0 or 16
    const bool hi8 = (lane & 8) != 0;
    float* tab = burst_lds + 2 * L::PART + wave * L::TAB;       // [2][GW][16]: scales, then biases
    const int esz = a.out_f32 ? 4 : 2;

    auto compute = [&](int64_t j, const BurstStage<BITS, GW>& st) __attribute__((always_inline)) {
        // the scales as floats, [group][row], for the accumulator lanes to
        // read 4 rows at a time (lane (c, r) holds row r, groups 2c, 2c + 1)
        tab[(2 * c) * 16 + r] = __uint_as_float(st.sw[0] << 16);
        tab[(2 * c + 1) * 16 + r] = __uint_as_float(st.sw[0] & 0xFFFF0000u);
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < G::KPW; ++p) {
            // pc[0][t]: codes of k-step t of the block, pc[1][t]: k-step 4 + t
            uint32_t pc[2][4];
            if constexpr (!NAT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t l0 = st.cw[8 * p + i], l1 = st.cw[8 * p + 4 + i];
                    const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0, 0x128, 0xF, 0xF, false);
                    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1, 0x128, 0xF, 0xF, false);
                    pc[0][i] = hi8 ? r1 : l0;
                    pc[1][i] = hi8 ? l1 : r0;
                }
                transpose4x4_rows(pc[0]);
                transpose4x4_rows(pc[1]);
            }
            constexpr int NG = NAT ? GW : G::GPK;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int g = NAT ? gi : p * G::GPK + gi;
                u32x4_t A0, A1, H0, H1;
                if constexpr (NAT) {
                    uint32_t w[NWN];
#pragma unroll
                    for (int q = 0; q + 1 < NWN; ++q)
                        w[q] = __builtin_amdgcn_alignbit(st.cw[g * NWN + q + 1], st.cw[g * NWN + q], wsh);
                    w[NWN - 1] = st.cw[g * NWN + NWN - 1] >> wsh;
                    A0 = codes_window_to_bf16<BITS, 0>(w, cmask, cmaskh, cbias);
                    A1 = codes_window_to_bf16<BITS, 1>(w, cmask, cmaskh, cbias);
                } else if constexpr (BITS == 4) {
                    A0 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1)], cmask, cbias);
                    A1 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1) + 1], cmask, cbias);
                } else if constexpr (BITS == 2) {
                    A0 = codes2_to_bf16(pc[gi >> 2][gi & 3], 0, cmask, cbias);
                    A1 = codes2_to_bf16(pc[gi >> 2][gi & 3], 1, cmask, cbias);
                } else {
                    codes8_to_bf16(pc[gi][0], pc[gi][1], cmask, cbias, A0, H0);
                    codes8_to_bf16(pc[gi][2], pc[gi][3], cmask, cbias, A1, H1);
                }
                f32x4_t dg = mfma16x16x32(A0, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
                dg = mfma16x16x32(A1, xb[2 * g + 1], dg);
                if constexpr (BITS == 8) {
                    f32x4_t dh = mfma16x16x32(H0, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
                    dh = mfma16x16x32(H1, xb[2 * g + 1], dh);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dg[i] = fmaf(16.0f, dh[i], dg[i]);
                }
                // read through the same pointer as the writes above
                const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(tab + g * 16 + 4 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc[i], dg[i] - z0[g], acc[i]);
            }
        }
        // + sum_g bias X_g: the rows' biases of groups 2c, 2c + 1 in slots
        // matching the pieces operand
        {
            const uint32_t bw = st.bw[0];
            const u32x4_t ab = u32x4_t{(bw & 0xFFFFu) | (bw << 16), bw, (bw >> 16) | (bw & 0xFFFF0000u), 0u};
            acc = mfma16x16x32(ab, bx, acc);
        }
        // partial tile into area j % 2; the barrier also orders this tile's
        // writes after every reader of the area two tiles back
        float* part = burst_lds + (j & 1) * L::PART;
#pragma unroll
        for (int i = 0; i < 4; ++i) part[(wave * 4 + i) * 65 + lane] = acc[i];
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        barrier_only();
        // output (m, n0 + n16) lives in lane (n16 / 4) * 16 + m, element
        // n16 % 4 of every wavefront's partial; summed in wavefront order
        const int tid = threadIdx.x;
        if (tid < 256) {
            const int m = tid >> 4, n16 = tid & 15;
            const int j0 = (n16 & 3) * 65 + (n16 >> 2) * 16 + m;
            float v = part[j0];
#pragma unroll
            for (int w = 1; w < NWV; ++w) v += part[w * 4 * 65 + j0];
            const int64_t n = (first + j * stride) * 16 + n16;
            if (m < a.M && n < a.N) {
                const size_t oi = (size_t)m * a.N + n;
                if (esz == 4) reinterpret_cast<float*>(a.y)[oi] = v;
                else reinterpret_cast<uint16_t*>(a.y)[oi] = f32_to_bf16_rne(v);
            }
        }
    };

    // every tile of the workgroup, computed in order (at most NT; the host
    // sizes the grid so)
    static_for<0, NT>([&](auto Uc) __attribute__((always_inline)) {
        constexpr int u = decltype(Uc)::value;
        if (u < ntile) compute(u, slot[u]);   // uniform over the workgroup
    });
}

// (bits, K) pairs served: K = 4096 with 8 wavefronts of 8 groups, 2..8 bits.
inline bool affine_burst_width(int bits, int K) { return K == 4096 && bits >= 2 && bits <= 8; }

// Offsets of every row the kernel addresses (up to one tile past N) fit the
// 32-bit buffer range.
inline bool affine_burst_supported(int bits, int N, int K)
{
    if (!affine_burst_width(bits, K)) return false;
    const int64_t rowb = (int64_t)K * bits / 8;
    return ((int64_t)N + 32) * rowb < 0x7FFFFFF0 && ((int64_t)N + 32) * (K / 64) * 2 < 0x7FFFFFF0;
}

// At most this many tiles per workgroup (all in flight at once).
constexpr int kAffineBurstMaxTiles = 4;

// One workgroup per CU (as many as fit), at least ceil(T / 4) so that no
// workgroup has more than 4 tiles; the instantiation with the fewest slots
// that holds a workgroup's tiles (1, 2 or 4), so no load is spent on slots
// that stay empty everywhere.
template <int BITS, int GW, int NWV>
hipError_t launch_affine_burst_one(const ProjArgs& a, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&affine_burst_kernel<BITS, GW, NWV, 4>);
    const size_t lds = BurstLds<GW, NWV>::BYTES;
    int cus = 0, bpc = 0;
    hipError_t e = device_cus(cus);
    if (e == hipSuccess) e = occupancy(bpc, fn, 64 * NWV, lds);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    int64_t blocks = (int64_t)bpc * cus;
    if (blocks > T) blocks = T;
    const int64_t need = (T + kAffineBurstMaxTiles - 1) / kAffineBurstMaxTiles;
    if (blocks < need) blocks = need;
    const int64_t per = (T + blocks - 1) / blocks;
    const dim3 grid((unsigned)blocks), block(64 * NWV);
    if (per == 1) hipLaunchKernelGGL((affine_burst_kernel<BITS, GW, NWV, 1>), grid, block, lds, s, a);
    else if (per == 2) hipLaunchKernelGGL((affine_burst_kernel<BITS, GW, NWV, 2>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((affine_burst_kernel<BITS, GW, NWV, 4>), grid, block, lds, s, a);
    return hipGetLastError();
}

// M = 17..32: one launch per 16-column half (rows 16.. of x and y).
template <int BITS>
hipError_t launch_affine_burst_impl(const ProjArgs& a, hipStream_t s)
{
    if (a.M > 32 || !affine_burst_supported(BITS, a.N, a.K)) return hipErrorInvalidValue;
    if (a.M <= 16) return launch_affine_burst_one<BITS, 8, 8>(a, s);
    ProjArgs lo = a, hi = a;
    lo.M = 16;
    hi.M = a.M - 16;
    hi.x = a.x + (size_t)16 * a.K;
    hi.y = static_cast<char*>(a.y) + (size_t)16 * a.N * (a.out_f32 ? 4 : 2);
    hipError_t e = launch_affine_burst_one<BITS, 8, 8>(lo, s);
    if (e == hipSuccess) e = launch_affine_burst_one<BITS, 8, 8>(hi, s);
    return e;
}

}  // namespace detail
}  // namespace aqg
