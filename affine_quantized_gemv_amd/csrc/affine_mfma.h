// Matrix-core kernel for 4-bit affine GEMVs at M = 3..32 (M padded to 16 or
// 32) on gfx950, for large N: persistent over 16-row tiles like
// mfma_stream.h.
//
// y^T[N, M] = W[N, K] . x^T[K, M] with W = scale * q + bias per 64-code
// group.  The A operand of v_mfma_f32_16x16x32_bf16 is built from the codes
// themselves: a field placed in a bf16 mantissa with 0x4300 gives exactly
// 128 + q (mask placement, no lookup), so one group's MFMA result is
// D = sum_k (128 + q_k) x_k, and the group contributes
// scale * D + (bias - 128 * scale) * X with X = sum_k x_k -- the exact
// factored form of sum_k x_k (scale * q_k + bias), in fp32.
//
// Operand flow per 128-byte k-block of the tile's 16 rows (256 codes per row):
//   * two buffer loads cover rows 0..7 and 8..15 with whole 128-byte lines,
//     and a row_ror:8 DPP select gives each lane one 16-byte piece of its
//     row (as in mfma_stream.h): lane (g, j) holds piece g (then 4 + g) of
//     row j, i.e. 32 codes of one half-group;
//   * a 4 x 4 transpose across the four 16-lane rows (v_permlane32_swap then
//     v_permlane16_swap) turns piece t into MFMA k-step t: lane (c, j) gets
//     dword c of piece t, codes 8c .. 8c + 7 of that k-step;
//   * each dword becomes four bf16 pairs (codes (0,4), (1,5), (2,6), (3,7)),
//     and x^T is staged in LDS in the same order, so the products pair up;
//   * two k-steps (one group) accumulate into a fresh 16 x 16 tile, which the
//     group's scale (from a small wavefront-private LDS table filled from one
//     bf16 load per lane per k-block) adds into the tile's sum in fp32;
//   * the bias and the 128 offset of the codes do not depend on the codes:
//     over the whole tile they are sum_g bias_g X_g - 128 sum_g scale_g X_g,
//     two small contractions over the groups that the matrix core also does
//     at the end of each tile (A = the tile's biases or scales, bf16, staged
//     per row in LDS; B = the group sums X split into bf16 high and low parts,
//     X - hi(X) being exact in bf16 to within 2^-16 of X).
// Codes of one group never mix with another group's in an MFMA, and each
// output is the same chain of MFMAs and fp32 operations for every M.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).
#pragma once
#include "mfma_stream.h"

namespace aqg {
namespace detail {

constexpr int kAffineMfmaThreads = 512;

// 4 x 4 transpose of dwords across the four 16-lane rows: on return v[t] at
// lane (row c, j) holds what v[c] held at lane (row t, j).
__device__ __forceinline__ void transpose4x4_rows(uint32_t (&v)[4])
{
    auto p0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    auto p1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    auto q0 = __builtin_amdgcn_permlane16_swap(p0[0], p1[0], false, false);
    auto q1 = __builtin_amdgcn_permlane16_swap(p0[1], p1[1], false, false);
    v[0] = q0[0]; v[1] = q0[1]; v[2] = q1[0]; v[3] = q1[1];
}

// Eight 4-bit codes (one dword, code i at bits 4i) -> bf16 pairs (128 + q):
// (q0, q4), (q1, q5), (q2, q6), (q3, q7).  m = 0x000F000F and c = 0x43004300
// come in as opaque registers so that plain C gives one v_and_or_b32 each.
// These values feed MFMA operands: they must come from instructions the
// compiler emits itself, since it only inserts the wait states an MFMA needs
// after a VALU write of its source registers for writes it can see (a write
// made inside inline asm is invisible to it).
__device__ __forceinline__ u32x4_t codes4_to_bf16(uint32_t w, uint32_t m, uint32_t c)
{
    return u32x4_t{(w & m) | c, ((w >> 4) & m) | c, ((w >> 8) & m) | c, ((w >> 12) & m) | c};
}

// LDS bytes private to one wavefront: the k-block's scales (bf16, 4 x 16)
// and the tile's bias and scale tables (bf16, 16 rows x 32-group multiples).
__host__ __device__ inline size_t affine_mfma_wave_bytes(int K)
{
    const int gps = ((K / 64 + 31) / 32) * 32;
    return 256 + (size_t)2 * 16 * gps * 2;
}

template <int MT, int D, int KSG>
__global__ void __launch_bounds__(kAffineMfmaThreads) affine4_mfma_kernel(ProjArgs a)
{
    extern __shared__ u32x4_t lds_a4[];
    constexpr int NB = MT / 16;
    constexpr int NW = kAffineMfmaThreads / 64;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;
    const int r = lane & 15;
    const int KS = a.K / 32;             // k-steps per row
    const int KBL = a.K / 256;           // 128-byte k-blocks per row (4 groups each)
    const int gpr = a.K / 64;
    // KSG: 32-group steps of the bias contractions (ceil(gpr / 32), a
    // template parameter so that the tile-end code has no loop of its own)
    constexpr int GPS = KSG * 32;        // groups per row in the bias tables (zero past gpr)
    const int64_t row_bytes = (int64_t)a.K / 2;
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

    // LDS: x^T fragments [s][b][lane]; X hi/lo fragments [ks][b][2][lane];
    // group sums [g][m] (prologue only); then per wavefront: scales of the
    // k-block in use [group][row], bias and scale tables [row][GPS] (all
    // bf16).
    u32x4_t* xb = lds_a4;
    u32x4_t* xh = xb + (size_t)KS * NB * 64;
    float* xs = reinterpret_cast<float*>(xh + (size_t)KSG * NB * 2 * 64);
    char* wbase = reinterpret_cast<char*>(xs + (size_t)gpr * MT) +
                  (size_t)wave * affine_mfma_wave_bytes(a.K);
    uint16_t* sbuf = reinterpret_cast<uint16_t*>(wbase);                        // [4][16] bf16
    uint16_t* btab = reinterpret_cast<uint16_t*>(wbase + 256);                  // [16][GPS]
    uint16_t* stab = btab + 16 * GPS;                                           // [16][GPS]

    // ---- ring of D k-blocks: two whole-line loads + one scale and one bias
    // per lane (lane l: row l/4, group l%4 of the k-block)
    u32x4_t wa[D][2];
    uint32_t sw[D], bw[D];
    int64_t f_tile = wg * CT;
    int f_c = 0;
    int f_b = 0;
    const int h = lane & 15;
    const uint32_t voff = (uint32_t)((h & 7) * row_bytes + 16 * ((h < 8 ? 0 : 4) + c));
    const int half_off = (int)(8 * row_bytes);
    const uint32_t goff = (uint32_t)(((lane >> 2) * gpr + (lane & 3)) * 2);
    auto fetch = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        const int64_t n0 = f_tile * 16;
        const int64_t rows = a.N - n0;
        const __amdgpu_buffer_rsrc_t rw = tile_rsrc(static_cast<const char*>(a.w0) + n0 * row_bytes, rows * row_bytes);
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.scales + n0 * gpr, rows * gpr * 2);
        const __amdgpu_buffer_rsrc_t rb = tile_rsrc(a.biases + n0 * gpr, rows * gpr * 2);
        sw[d] = __builtin_amdgcn_raw_buffer_load_b16(rs, goff, 8 * f_b, kLoadNT);
        bw[d] = __builtin_amdgcn_raw_buffer_load_b16(rb, goff, 8 * f_b, kLoadNT);
        wa[d][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, 128 * f_b, kLoadNT));
        wa[d][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, 128 * f_b + half_off, kLoadNT));
        const bool wrap = f_b + 1 == KBL;
        const bool stw = wrap && f_c + 1 == CT;
        f_b = wrap ? 0 : f_b + 1;
        f_c = wrap ? (stw ? 0 : f_c + 1) : f_c;
        f_tile += wrap ? (stw ? (W - 1) * CT + 1 : 1) : 0;
    };

    f32x4_t acc[NB], accb[NB], accs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = accb[b] = accs[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int c_b = 0;
    int64_t c_tile = wg * CT;            // tile being consumed
    int c_c = 0;                         // its index within the super-tile
    const bool hi8 = (lane & 8) != 0;
    uint32_t cmask = 0x000F000Fu, cbias = 0x43004300u;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+v"(cbias));

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        // the k-block's scales and biases into the wavefront's tables (LDS
        // operations of one wavefront take effect in program order)
        {
            // raw 16-bit values straight from the loads: arithmetic on them
            // here would be hoisted into the loop latch and wait there
            sbuf[(lane & 3) * 16 + (lane >> 2)] = (uint16_t)sw[d];
            const int ti2 = (lane >> 2) * GPS + 4 * c_b + (lane & 3);
            btab[ti2] = (uint16_t)bw[d];
            stab[ti2] = (uint16_t)sw[d];
        }
        // pieces: s[0] = pieces 0..3 of row j in lane-row g, s[1] = pieces 4..7
        uint32_t pc[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l0 = wa[d][0][i], l1 = wa[d][1][i];
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0, 0x128, 0xF, 0xF, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1, 0x128, 0xF, 0xF, false);
            pc[0][i] = hi8 ? r1 : l0;
            pc[1][i] = hi8 ? l1 : r0;
        }
        transpose4x4_rows(pc[0]);        // pc[0][t]: codes of k-step t of the block
        transpose4x4_rows(pc[1]);        // pc[1][t]: k-step 4 + t
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            // scales of rows 4c .. 4c + 3, group gi
            const uint2 s4 = *reinterpret_cast<const uint2*>(sbuf + gi * 16 + 4 * c);
            const float sc[4] = {__uint_as_float(s4.x << 16), __uint_as_float(s4.x & 0xFFFF0000u),
                                 __uint_as_float(s4.y << 16), __uint_as_float(s4.y & 0xFFFF0000u)};
            const u32x4_t A0 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1)], cmask, cbias);
            const u32x4_t A1 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1) + 1], cmask, cbias);
            const int S0 = 8 * c_b + 2 * gi;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4_t dg = mfma16x16x32(A0, xb[(S0 * NB + b) * 64 + lane], f32x4_t{0.f, 0.f, 0.f, 0.f});
                dg = mfma16x16x32(A1, xb[((S0 + 1) * NB + b) * 64 + lane], dg);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[b][i] = fmaf(sc[i], dg[i], acc[b][i]);
            }
        }
        if (++c_b == KBL) {
            // end of the tile: bias and code-offset terms, then stage
            c_b = 0;
#pragma unroll
            for (int ks = 0; ks < KSG; ++ks) {
                const u32x4_t Ab = *reinterpret_cast<const u32x4_t*>(btab + r * GPS + 32 * ks + 8 * c);
                const u32x4_t As = *reinterpret_cast<const u32x4_t*>(stab + r * GPS + 32 * ks + 8 * c);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const u32x4_t Xh = xh[((ks * NB + b) * 2 + 0) * 64 + lane];
                    const u32x4_t Xl = xh[((ks * NB + b) * 2 + 1) * 64 + lane];
                    accb[b] = mfma16x16x32(Ab, Xh, accb[b]);
                    accb[b] = mfma16x16x32(Ab, Xl, accb[b]);
                    accs[b] = mfma16x16x32(As, Xh, accs[b]);
                    accs[b] = mfma16x16x32(As, Xl, accs[b]);
                }
            }
            // lane (c, r) holds rows 4c .. 4c + 3 of column 16b + r: store
            // them now (no staging: either way consecutive lanes write
            // different rows of y)
            const int64_t n0 = c_tile * 16 + 4 * c;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int m = 16 * b + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = fmaf(-128.0f, accs[b][i], acc[b][i] + accb[b][i]);
                    if (m < a.M && n0 + i < a.N) {
                        const size_t o = (size_t)m * a.N + (size_t)(n0 + i);
                        if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = v;
                        else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(v);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = accb[b] = accs[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // next tile of this wavefront
            ++c_c;
            if (c_c == CT) { c_c = 0; c_tile += (W - 1) * CT + 1; } else { ++c_tile; }
        }
    };

    // prologue: D k-blocks, then stage x^T (pair order within each 8-k chunk),
    // the group sums X, their bf16 high/low fragments, and clear the bias
    // tables (groups past gpr stay zero)
    static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(Dd); });
    {
        constexpr int XB = 4;
        const int ntask = KS * NB * 64;
        for (int t0 = threadIdx.x; t0 < ntask; t0 += XB * kAffineMfmaThreads) {
            u32x4_t v[XB];
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kAffineMfmaThreads;
                const int l = t & 63;
                const int sb = t >> 6;
                const int s = sb / NB, b = sb - s * NB;
                const int m = 16 * b + (l & 15);
                v[i] = u32x4_t{0u, 0u, 0u, 0u};
                if (t < ntask && m < a.M)
                    v[i] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)m * a.K + 32 * s + 8 * (l >> 4));
            }
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kAffineMfmaThreads;
                if (t < ntask) {
                    // x words (x0|x1), (x2|x3), (x4|x5), (x6|x7) -> (x0|x4), (x1|x5), (x2|x6), (x3|x7)
                    const uint32_t w0 = v[i][0], w1 = v[i][1], w2 = v[i][2], w3 = v[i][3];
                    xb[t] = u32x4_t{(w0 & 0xFFFFu) | (w2 << 16), (w0 >> 16) | (w2 & 0xFFFF0000u),
                                    (w1 & 0xFFFFu) | (w3 << 16), (w1 >> 16) | (w3 & 0xFFFF0000u)};
                }
            }
        }
        for (int t = threadIdx.x; t < gpr * MT; t += kAffineMfmaThreads) {
            const int g = t / MT, m = t - g * MT;
            float sum = 0.0f;
            if (m < a.M) {
                const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)m * a.K + 64 * g);
                float part[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 q = src[i];
                    part[i] = ((bf16_to_f32(q.x & 0xFFFFu) + bf16_to_f32(q.x >> 16)) +
                               (bf16_to_f32(q.y & 0xFFFFu) + bf16_to_f32(q.y >> 16))) +
                              ((bf16_to_f32(q.z & 0xFFFFu) + bf16_to_f32(q.z >> 16)) +
                               (bf16_to_f32(q.w & 0xFFFFu) + bf16_to_f32(q.w >> 16)));
                }
                sum = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
            }
            xs[t] = sum;
        }
        for (int t = lane; t < 2 * 16 * GPS / 2; t += 64)          // both tables, as 32-bit words
            reinterpret_cast<uint32_t*>(btab)[t] = 0u;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < KSG * NB * 64; t += kAffineMfmaThreads) {
        // X fragment: lane (c, col) of block b holds groups 32ks + 8c .. + 7 of column 16b + col
        const int l = t & 63;
        const int kb = t >> 6;
        const int ks = kb / NB, b = kb - ks * NB;
        const int m = 16 * b + (l & 15);
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t hh[2], ll[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int g = 32 * ks + 8 * (l >> 4) + 2 * j + e;
                const float X = g < gpr ? xs[g * MT + m] : 0.0f;
                const uint16_t hb = f32_to_bf16_rne(X);
                hh[e] = hb;
                ll[e] = f32_to_bf16_rne(X - bf16_to_f32(hb));
            }
            hw[j] = hh[0] | (hh[1] << 16);
            lw[j] = ll[0] | (ll[1] << 16);
        }
        xh[(kb * 2 + 0) * 64 + l] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
        xh[(kb * 2 + 1) * 64 + l] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    }
    // Every load issued so far is complete (the x loads came after the
    // weights and loads complete in order); saying so keeps a possibly
    // pending staging load out of the loop's waits.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (my_tiles == 0) return;

    const int64_t nitems = my_tiles * KBL;
    int64_t base = 0;
    for (; base + 2 * D <= nitems; base += D) {
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            consume(Dd);
            fetch(Dd);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    for (; base < nitems; base += D) {
        static_for<0, D>([&](auto Dd) __attribute__((always_inline)) {
            constexpr int d = decltype(Dd)::value;
            if (base + d < nitems) {
                consume(Dd);
                if (base + d + D < nitems) fetch(Dd);
            }
        });
    }

}

// k-blocks in flight per wavefront and workgroups per CU: on the 151936 x
// 1024 LM head at M = 16, depth 4 with 2 workgroups (16 wavefronts) per CU
// measured fastest (3 workgroups, i.e. more bytes in flight, ~20% slower).
constexpr int kAffineMfmaDepth = 4;
constexpr int kAffineMfmaWgPerCu = 2;

inline size_t affine_mfma_lds_bytes(int MT, int K)
{
    const int gpr = K / 64, ksg = (gpr + 31) / 32;
    return (size_t)(K / 32) * (MT / 16) * 64 * 16 + (size_t)ksg * (MT / 16) * 2 * 64 * 16 + (size_t)gpr * MT * 4 +
           (size_t)(kAffineMfmaThreads / 64) * affine_mfma_wave_bytes(K);
}

template <int MT, int KSG>
hipError_t launch_affine_mfma_one(const ProjArgs& a, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&affine4_mfma_kernel<MT, kAffineMfmaDepth, KSG>);
    {
        static std::atomic<int> raised{0};
        if (!raised.load(std::memory_order_acquire)) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfmaStreamLdsMax);
            if (e != hipSuccess) return e;
            raised.store(1, std::memory_order_release);
        }
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    constexpr int NW = kAffineMfmaThreads / 64;
    const size_t lds = affine_mfma_lds_bytes(MT, a.K);
    if (lds > kMfmaStreamLdsMax) return hipErrorInvalidValue;
    int bpc = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, fn, kAffineMfmaThreads, lds);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    if (bpc > kAffineMfmaWgPerCu) bpc = kAffineMfmaWgPerCu;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    int64_t waves = (int64_t)bpc * cus * NW;
    if (waves > T) waves = T;
    const int blocks = (int)((waves + NW - 1) / NW);
    ProjArgs a2 = a;
    a2.tpw = 1;
    hipLaunchKernelGGL((affine4_mfma_kernel<MT, kAffineMfmaDepth, KSG>), dim3(blocks), dim3(kAffineMfmaThreads), lds, s, a2);
    return hipGetLastError();
}

inline hipError_t launch_affine_mfma_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    const int ksg = (a.K / 64 + 31) / 32;
    if (ksg == 1) return c.MT == 16 ? launch_affine_mfma_one<16, 1>(a, s) : launch_affine_mfma_one<32, 1>(a, s);
    if (ksg == 2) return c.MT == 16 ? launch_affine_mfma_one<16, 2>(a, s) : launch_affine_mfma_one<32, 2>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace detail
}  // namespace aqg
