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

// Groups per row of a K-chunk's tables: the chunk's groups (K/256 k-blocks
// split into nkc chunks of at most ceil(K/256 / nkc) blocks, 4 groups each)
// rounded up to 8, 16, 32 or 64.
inline int affine_mfma_gps(int K, int nkc)
{
    const int g = 4 * ((K / 256 + nkc - 1) / nkc);
    return g <= 8 ? 8 : g <= 16 ? 16 : g <= 32 ? 32 : g <= 64 ? 64 : 0;
}

// LDS bytes private to one wavefront: the k-block's scales (bf16, 4 x 16)
// and its chunk's bias and scale tables (bf16, 16 rows x gps).
__host__ __device__ inline size_t affine_mfma_wave_bytes(int gps)
{
    return 256 + (size_t)2 * 16 * gps * 2;
}

template <int MT, int D, int GPS>
__global__ void __launch_bounds__(kAffineMfmaThreads) affine4_mfma_kernel(ProjArgs a)
{
    extern __shared__ u32x4_t lds_a4[];
    constexpr int NB = MT / 16;
    constexpr int NW = kAffineMfmaThreads / 64;
    constexpr int PER_TILE = 16 * MT;
    // GPS: groups per row in a chunk's tables (zero past the chunk's end);
    // the bias contractions take 32 groups per step (KSG steps) and only the
    // first LV lanes of their operands can be non-zero
    constexpr int KSG = (GPS + 31) / 32;
    constexpr int LV = GPS * 2 < 64 ? GPS * 2 : 64;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;
    const int r = lane & 15;
    const int KS = a.K / 32;             // k-steps per row
    const int KBL = a.K / 256;           // 128-byte k-blocks per row (4 groups each)
    const int gpr = a.K / 64;
    const int64_t row_bytes = (int64_t)a.K / 2;
    const int64_t T = ((int64_t)a.N + 15) / 16;

    // K split: wavefront w of a workgroup takes chunk j = w % nkc of the
    // k-blocks of the tiles of its slot s = w / nkc; the slots of all
    // workgroups take the row tiles round-robin
    const int lk = a.ksplit_log2;
    const int nkc = 1 << lk;
    const int j = wave & (nkc - 1);
    const int TS = NW >> lk;
    const int kb_lo = j * KBL / nkc, kb_hi = (j + 1) * KBL / nkc;
    const int64_t U = (int64_t)gridDim.x * TS;
    const int64_t u = (int64_t)blockIdx.x * TS + (wave >> lk);
    const int64_t my_tiles = u < T ? (T - 1 - u) / U + 1 : 0;

    // LDS: x^T fragments [s][b][lane]; X hi/lo fragments [chunk][ks][b][2][lane];
    // sums of x per (k-step, column) (prologue only); per wavefront:
    // scales of the k-block
    // in use [group][row], its chunk's bias and scale tables [row][GPS] (all
    // bf16); with a K split, the chunks' partial tiles [slot][tile][chunk].
    u32x4_t* xb = lds_a4;
    u32x4_t* xh = xb + (size_t)KS * NB * 64;
    float* xs = reinterpret_cast<float*>(xh + (size_t)nkc * KSG * NB * 2 * LV);
    char* wbase0 = reinterpret_cast<char*>(xs + (size_t)KS * MT);
    char* wbase = wbase0 + (size_t)wave * affine_mfma_wave_bytes(GPS);
    uint16_t* sbuf = reinterpret_cast<uint16_t*>(wbase);                        // [4][16] bf16
    uint16_t* btab = reinterpret_cast<uint16_t*>(wbase + 256);                  // [16][GPS]
    uint16_t* stab = btab + 16 * GPS;                                           // [16][GPS]
    float* pbuf = reinterpret_cast<float*>(wbase0 + (size_t)NW * affine_mfma_wave_bytes(GPS));

    // ---- ring of D k-blocks: two whole-line loads + one scale and one bias
    // per lane (lane l: row l/4, group l%4 of the k-block)
    u32x4_t wa[D][2];
    uint32_t sw[D], bw[D];
    int64_t f_tile = u;
    int f_b = kb_lo;
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
        const bool wrap = f_b + 1 == kb_hi;
        f_b = wrap ? kb_lo : f_b + 1;
        f_tile += wrap ? U : 0;
    };

    f32x4_t acc[NB], accb[NB], accs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = accb[b] = accs[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int c_b = kb_lo;                     // k-block being consumed
    int64_t c_tile = u;                  // its tile
    int ti = 0;                          // tiles finished (K split: partials staged)
    const bool hi8 = (lane & 8) != 0;
    uint32_t cmask = 0x000F000Fu, cbias = 0x43004300u;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+v"(cbias));
    const u32x4_t* xhj = xh + (size_t)j * KSG * NB * 2 * LV;

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        // the k-block's scales and biases into the wavefront's tables (LDS
        // operations of one wavefront take effect in program order)
        {
            // raw 16-bit values straight from the loads: arithmetic on them
            // here would be hoisted into the loop latch and wait there
            sbuf[(lane & 3) * 16 + (lane >> 2)] = (uint16_t)sw[d];
            const int ti2 = (lane >> 2) * GPS + 4 * (c_b - kb_lo) + (lane & 3);
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
        if (++c_b == kb_hi) {
            // end of the tile (or of its K-chunk): bias and code-offset terms
            c_b = kb_lo;
            const bool lv = lane < LV;
#pragma unroll
            for (int ks = 0; ks < KSG; ++ks) {
                const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
                const u32x4_t Ab = lv ? *reinterpret_cast<const u32x4_t*>(btab + r * GPS + 32 * ks + 8 * c) : z;
                const u32x4_t As = lv ? *reinterpret_cast<const u32x4_t*>(stab + r * GPS + 32 * ks + 8 * c) : z;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const u32x4_t Xh = lv ? xhj[((ks * NB + b) * 2 + 0) * LV + lane] : z;
                    const u32x4_t Xl = lv ? xhj[((ks * NB + b) * 2 + 1) * LV + lane] : z;
                    accb[b] = mfma16x16x32(Ab, Xh, accb[b]);
                    accb[b] = mfma16x16x32(Ab, Xl, accb[b]);
                    accs[b] = mfma16x16x32(As, Xh, accs[b]);
                    accs[b] = mfma16x16x32(As, Xl, accs[b]);
                }
            }
            // lane (c, r) holds rows 4c .. 4c + 3 of column 16b + r
            if (nkc == 1) {
                // whole tile: store now (staging would not coalesce either:
                // consecutive lanes write different rows of y)
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
            } else {
                float* pt = pbuf + ((((size_t)(wave >> lk) * a.tmax + ti) * nkc + j) * PER_TILE);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pt[(4 * c + i) * MT + 16 * b + r] = fmaf(-128.0f, accs[b][i], acc[b][i] + accb[b][i]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = accb[b] = accs[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            c_tile += U;
            ++ti;
        }
    };

    // prologue: D k-blocks, then stage x^T (pair order within each 8-k chunk)
    // with the sums of each staged 8 x, then each chunk's group sums X as
    // bf16 high/low fragments, and clear the bias tables (groups past the
    // chunk's end stay zero)
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
                    // sum of the k-step's 32 x of column m: this lane's 8,
                    // then across the four quarters (lanes 16 apart; the whole
                    // wavefront is here: ntask is a multiple of 64)
                    const int l = t & 63;
                    const int sb = t >> 6;
                    const int s = sb / NB, b = sb - s * NB;
                    const int m = 16 * b + (l & 15);
                    float p8 = ((bf16_to_f32(w0 & 0xFFFFu) + bf16_to_f32(w0 >> 16)) + (bf16_to_f32(w1 & 0xFFFFu) + bf16_to_f32(w1 >> 16))) +
                               ((bf16_to_f32(w2 & 0xFFFFu) + bf16_to_f32(w2 >> 16)) + (bf16_to_f32(w3 & 0xFFFFu) + bf16_to_f32(w3 >> 16)));
                    p8 += __shfl_xor(p8, 16);
                    p8 += __shfl_xor(p8, 32);
                    if (l < 16) xs[s * MT + m] = p8;
                }
            }
        }
        for (int t = lane; t < 16 * GPS; t += 64)          // both tables, as 32-bit words
            reinterpret_cast<uint32_t*>(btab)[t] = 0u;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < nkc * KSG * NB * LV; t += kAffineMfmaThreads) {
        // X fragment of chunk jj: lane (c, col) of block b holds the chunk's
        // groups 32ks + 8c .. + 7 of column 16b + col (lanes < LV only)
        const int l = t % LV;
        const int kb = t / LV;
        const int jj = kb / (KSG * NB);
        const int rem = kb - jj * (KSG * NB);
        const int ks = rem / NB, b = rem - ks * NB;
        const int m = 16 * b + (l & 15);
        const int g_lo = 4 * (jj * KBL / nkc), g_hi = 4 * ((jj + 1) * KBL / nkc);
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t hh[2], ll[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int g = g_lo + 32 * ks + 8 * (l >> 4) + 2 * q + e;
                // the group's 64 x: k-steps 2g and 2g + 1
                const float X = g < g_hi ? xs[(2 * g) * MT + m] + xs[(2 * g + 1) * MT + m] : 0.0f;
                const uint16_t hb = f32_to_bf16_rne(X);
                hh[e] = hb;
                ll[e] = f32_to_bf16_rne(X - bf16_to_f32(hb));
            }
            hw[q] = hh[0] | (hh[1] << 16);
            lw[q] = ll[0] | (ll[1] << 16);
        }
        xh[(kb * 2 + 0) * LV + l] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
        xh[(kb * 2 + 1) * LV + l] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    }
    // Every load issued so far is complete (the x loads came after the
    // weights and loads complete in order); saying so keeps a possibly
    // pending staging load out of the loop's waits.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // without a K split nothing below waits for the other wavefronts
    if (nkc == 1 && my_tiles == 0) return;

    const int64_t nitems = my_tiles * (kb_hi - kb_lo);
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
    if (nkc == 1) return;

    // K split: sum the chunks' partial tiles in chunk order and store
    __syncthreads();
    const int64_t nout = (int64_t)TS * a.tmax * PER_TILE;
    for (int64_t v = threadIdx.x; v < nout; v += kAffineMfmaThreads) {
        const int64_t st = v / PER_TILE;                 // slot * tmax + tile index
        const int rem = (int)(v - st * PER_TILE);
        const int sl = (int)(st / a.tmax), tix = (int)(st - (int64_t)sl * a.tmax);
        const int m = rem % MT;
        const int64_t tile = (int64_t)blockIdx.x * TS + sl + (int64_t)tix * U;
        const int64_t n = tile * 16 + rem / MT;
        if (tile < T && m < a.M && n < a.N) {
            const float* pt = pbuf + (size_t)st * nkc * PER_TILE + rem;
            float val = pt[0];
            for (int jj = 1; jj < nkc; ++jj) val += pt[(size_t)jj * PER_TILE];
            const size_t o = (size_t)m * a.N + n;
            if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = val;
            else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(val);
        }
    }
}

// k-blocks in flight per wavefront and workgroups per CU: on the 151936 x
// 1024 LM head at M = 16, depth 4 with 2 workgroups (16 wavefronts) per CU
// measured fastest (3 workgroups, i.e. more bytes in flight, ~20% slower).
constexpr int kAffineMfmaDepth = 4;
constexpr int kAffineMfmaWgPerCu = 2;

// LDS bytes of one workgroup with nkc K-chunks per tile and, for nkc > 1,
// tmax tiles per slot staged as partials.
inline size_t affine_mfma_lds_bytes(int MT, int K, int nkc, int64_t tmax)
{
    const int gps = affine_mfma_gps(K, nkc);
    const int ksg = (gps + 31) / 32, lv = gps * 2 < 64 ? gps * 2 : 64;
    const int nw = kAffineMfmaThreads / 64;
    size_t b = (size_t)(K / 32) * (MT / 16) * 64 * 16 + (size_t)nkc * ksg * (MT / 16) * 2 * lv * 16 +
               (size_t)(K / 32) * MT * 4 + (size_t)nw * affine_mfma_wave_bytes(gps);
    if (nkc > 1) b += (size_t)nw * tmax * 16 * MT * 4;
    return b;
}

// Launch geometry: workgroups and tiles per slot for nkc chunks per tile.
inline void affine_mfma_geometry(int64_t T, int nkc, int cus, int bpc, int& blocks, int64_t& tmax)
{
    const int ts = (kAffineMfmaThreads / 64) / nkc;
    int64_t slots = (int64_t)bpc * cus * ts;
    const int64_t need = T;                              // one tile per slot if possible
    if (slots > need) slots = need;
    blocks = (int)((slots + ts - 1) / ts);
    tmax = (T + (int64_t)blocks * ts - 1) / ((int64_t)blocks * ts);
}

template <int MT, int GPS>
hipError_t launch_affine_mfma_one(const ProjArgs& a, int nkc, hipStream_t s)
{
    const void* fn = reinterpret_cast<const void*>(&affine4_mfma_kernel<MT, kAffineMfmaDepth, GPS>);
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
    const int64_t T = ((int64_t)a.N + 15) / 16;
    int bpc = kAffineMfmaWgPerCu, blocks = 0;
    int64_t tmax = 0;
    size_t lds = 0;
    for (;;) {
        affine_mfma_geometry(T, nkc, cus, bpc, blocks, tmax);
        lds = affine_mfma_lds_bytes(MT, a.K, nkc, tmax);
        if (lds > kMfmaStreamLdsMax) return hipErrorInvalidValue;
        int occ = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kAffineMfmaThreads, lds);
        if (e != hipSuccess) return e;
        if (occ >= bpc || bpc == 1) break;
        bpc = occ < 1 ? 1 : occ;
    }
    ProjArgs a2 = a;
    a2.tpw = 1;
    a2.tmax = tmax;
    int lk = 0;
    while ((1 << lk) < nkc) ++lk;
    a2.ksplit_log2 = lk;
    hipLaunchKernelGGL((affine4_mfma_kernel<MT, kAffineMfmaDepth, GPS>), dim3(blocks), dim3(kAffineMfmaThreads), lds, s, a2);
    return hipGetLastError();
}

inline hipError_t launch_affine_mfma_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    const int nkc = 1 << c.ksplit_log2;
    if (nkc > kAffineMfmaThreads / 64 || nkc > a.K / 256) return hipErrorInvalidValue;   // every chunk >= 1 k-block
    const bool w = c.MT == 16;
    switch (affine_mfma_gps(a.K, nkc)) {
        case 8: return w ? launch_affine_mfma_one<16, 8>(a, nkc, s) : launch_affine_mfma_one<32, 8>(a, nkc, s);
        case 16: return w ? launch_affine_mfma_one<16, 16>(a, nkc, s) : launch_affine_mfma_one<32, 16>(a, nkc, s);
        case 32: return w ? launch_affine_mfma_one<16, 32>(a, nkc, s) : launch_affine_mfma_one<32, 32>(a, nkc, s);
        case 64: return w ? launch_affine_mfma_one<16, 64>(a, nkc, s) : launch_affine_mfma_one<32, 64>(a, nkc, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
