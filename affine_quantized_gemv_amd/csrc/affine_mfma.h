// Matrix-core kernel for affine GEMVs with 2-, 4- and 8-bit codes at M up
// to 32 (M padded to 16 or 32) on gfx950: persistent over 16-row tiles like
// mfma_stream.h, with the K range split over a workgroup's wavefronts when
// there are few tiles.
//
// y^T[N, M] = W[N, K] . x^T[K, M] with W = scale * q + bias per 64-code
// group.  The A operand of v_mfma_f32_16x16x32_bf16 is built from the codes
// themselves: a field placed in a bf16 mantissa with 0x4300 gives exactly
// 128 + q (mask placement, no lookup); 8-bit codes go in as two nibbles, the
// high one in a second MFMA chain weighted 16 in fp32.  So one group's result
// is D = sum_k (C + q_k) x_k with C = 128 (2176 for 8 bits), and the group
// contributes scale * (D - D0) + bias * X with X = sum_k x_k -- the factored
// form of sum_k x_k (scale * q_k + bias), in fp32.  D0 is the code offset
// C * X computed by the matrix core itself: the same two (or, for 8 bits,
// four) MFMAs on the same x^T operands with every code zero, once per group
// and column in the prologue.  A group whose codes are all zero thus gives
// D == D0 bit for bit and adds exactly bias * X (no residue of the offset).
//
// Operand flow per 128-byte k-block of the tile's 16 rows:
//   * two buffer loads cover rows 0..7 and 8..15 with whole 128-byte lines,
//     and a row_ror:8 DPP select gives each lane one 16-byte piece of its
//     row (as in mfma_stream.h);
//   * a 4 x 4 transpose across the four 16-lane rows (v_permlane32_swap then
//     v_permlane16_swap) leaves lane (c, r) with dword c of each of the
//     block's 8 pieces of row r;
//   * a group's 64 codes are 16 per lane (one dword at 2 bits, two at 4,
//     four at 8 bits); they become the A operands of two k-steps, and x^T is
//     staged in LDS with the matching k order, so the products pair up (the
//     k order inside a group is free: it only has to agree on both sides);
//   * the two k-steps of a group accumulate into a fresh 16 x 16 tile D; the
//     group's scale (from a small wavefront-private LDS table filled from the
//     scale loads) times D - D0 (D0 from an LDS table per group and column)
//     is added into the tile's sum in fp32;
//   * the bias term does not depend on the codes: over the tile it is
//     sum_g bias_g X_g, a small contraction over the groups that the matrix
//     core also does at the end of each tile (A = the tile's biases, bf16,
//     staged per row in LDS; B = the group sums X split into bf16 high and
//     low parts, X - hi(X) being exact in bf16 to within 2^-16 of X).
// Codes of one group never mix with another group's in an MFMA, and each
// output is the same chain of MFMAs and fp32 operations for every M of a
// 16-column bucket.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).
#pragma once
#include "argmax.h"
#include "mfma_stream.h"

namespace aqg {
namespace detail {

constexpr int kAffineMfmaThreads = 512;
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

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

// Sixteen 2-bit codes (code i at bits 2i) -> bf16 pairs (q_i, q_{i+8}) for
// i = 4h .. 4h + 3 (h = 0, 1): the A operands of the group's two k-steps.
// m = 0x00030003 and c = 0x43004300 as opaque registers.
__device__ __forceinline__ u32x4_t codes2_to_bf16(uint32_t w, int h, uint32_t m, uint32_t c)
{
    const uint32_t v = w >> (8 * h);
    return u32x4_t{(v & m) | c, ((v >> 2) & m) | c, ((v >> 4) & m) | c, ((v >> 6) & m) | c};
}

// Eight 8-bit codes, a0..a3 in dword a and b0..b3 in dword b (byte i = code
// i), as two nibble operands in the order (a0, a2), (a1, a3), (b0, b2),
// (b1, b3): lo holds 128 + the low nibbles, hi 128 + the high nibbles.
__device__ __forceinline__ void codes8_to_bf16(uint32_t a, uint32_t b, uint32_t m, uint32_t c, u32x4_t& lo, u32x4_t& hi)
{
    lo = u32x4_t{(a & m) | c, ((a >> 8) & m) | c, (b & m) | c, ((b >> 8) & m) | c};
    hi = u32x4_t{((a >> 4) & m) | c, ((a >> 12) & m) | c, ((b >> 4) & m) | c, ((b >> 12) & m) | c};
}

// Per-width geometry: groups per 128-byte k-block of a row, the code offset C
// of the A operands, and the field mask.
template <int BITS> struct AffineMma;
template <> struct AffineMma<2> { static constexpr int GPK = 8; static constexpr float OFF = 128.0f; static constexpr uint32_t MASK = 0x00030003u; };
template <> struct AffineMma<4> { static constexpr int GPK = 4; static constexpr float OFF = 128.0f; static constexpr uint32_t MASK = 0x000F000Fu; };
template <> struct AffineMma<8> { static constexpr int GPK = 2; static constexpr float OFF = 2176.0f; static constexpr uint32_t MASK = 0x000F000Fu; };

// k-blocks (128 bytes) per row.
inline int affine_mfma_kbl(int K, int bits) { return K * bits / 1024; }

// Groups per row of a K-chunk's tables: the chunk's groups (the row's
// k-blocks split into nkc chunks of at most ceil(kbl / nkc) blocks) rounded
// up to 8, 16, 32 or 64.
inline int affine_mfma_gps(int K, int bits, int nkc)
{
    const int kbl = affine_mfma_kbl(K, bits);
    const int g = (16 / bits) * ((kbl + nkc - 1) / nkc);
    return g <= 8 ? 8 : g <= 16 ? 16 : g <= 32 ? 32 : g <= 64 ? 64 : 0;
}

// Staged x^T operand of k-step S (group S / 2, half S % 2) for lane quarter
// c, in the k order of that width's A operands, from row xr of x; also the
// sum of its 8 values.
template <int BITS>
__device__ __forceinline__ u32x4_t stage_x_operand(const uint16_t* xr, int S, int c, float& sum)
{
    const int base = 64 * (S >> 1), t = S & 1;
    uint32_t o[4];
    if constexpr (BITS == 4) {
        // x at 32t + 8c + {0,4,1,5,2,6,3,7}
        const uint4 v = *reinterpret_cast<const uint4*>(xr + base + 32 * t + 8 * c);
        o[0] = (v.x & 0xFFFFu) | (v.z << 16); o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        o[2] = (v.y & 0xFFFFu) | (v.w << 16); o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
    } else if constexpr (BITS == 2) {
        // x at 16c + 4t + {0,8,1,9,2,10,3,11}
        const uint2 p = *reinterpret_cast<const uint2*>(xr + base + 16 * c + 4 * t);
        const uint2 q = *reinterpret_cast<const uint2*>(xr + base + 16 * c + 4 * t + 8);
        o[0] = (p.x & 0xFFFFu) | (q.x << 16); o[1] = (p.x >> 16) | (q.x & 0xFFFF0000u);
        o[2] = (p.y & 0xFFFFu) | (q.y << 16); o[3] = (p.y >> 16) | (q.y & 0xFFFF0000u);
    } else {
        // x at 32t + 4c + {0,2,1,3, 16,18,17,19}
        const uint2 p = *reinterpret_cast<const uint2*>(xr + base + 32 * t + 4 * c);
        const uint2 q = *reinterpret_cast<const uint2*>(xr + base + 32 * t + 4 * c + 16);
        o[0] = (p.x & 0xFFFFu) | (p.y << 16); o[1] = (p.x >> 16) | (p.y & 0xFFFF0000u);
        o[2] = (q.x & 0xFFFFu) | (q.y << 16); o[3] = (q.x >> 16) | (q.y & 0xFFFF0000u);
    }
    sum = ((bf16_to_f32(o[0] & 0xFFFFu) + bf16_to_f32(o[0] >> 16)) + (bf16_to_f32(o[1] & 0xFFFFu) + bf16_to_f32(o[1] >> 16))) +
          ((bf16_to_f32(o[2] & 0xFFFFu) + bf16_to_f32(o[2] >> 16)) + (bf16_to_f32(o[3] & 0xFFFFu) + bf16_to_f32(o[3] >> 16)));
    return u32x4_t{o[0], o[1], o[2], o[3]};
}

// LDS bytes private to one wavefront: the k-block's scales (bf16, 4 x 16)
// and its chunk's bias table (bf16, 16 rows x gps).
__host__ __device__ inline size_t affine_mfma_wave_bytes(int gps)
{
    return 256 + (size_t)16 * gps * 2;
}

// XR: the x^T operands and code offsets of the whole row held in registers
// (4-bit codes, K = 1024, 16 columns, no K split: then the ring's slot d
// always holds k-block d of a tile, so they are indexed with constants).
template <int BITS, int MT, int D, int GPS, bool XR>
__global__ void __launch_bounds__(kAffineMfmaThreads) affine_mfma_kernel(ProjArgs a)
{
    extern __shared__ u32x4_t lds_a4[];
    constexpr int XRS = XR ? 32 : 1;   // k-steps held in registers
    static_assert(!XR || (BITS == 4 && MT == 16 && D == 4), "register x: 4-bit codes, K = 1024, 16 columns");
    constexpr int NB = MT / 16;
    constexpr int NW = kAffineMfmaThreads / 64;
    constexpr int PER_TILE = 16 * MT;
    constexpr int GPK = AffineMma<BITS>::GPK;   // groups per 128-byte k-block
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
    const int KBL = a.K * BITS / 1024;   // 128-byte k-blocks per row (GPK groups each)
    const int gpr = a.K / 64;
    const int64_t row_bytes = (int64_t)a.K * BITS / 8;
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
    // sums of x per (k-step, column) in the prologue, then the code offsets
    // D0 per (group, column); per wavefront: scales of the k-block in use
    // [group][row] and its chunk's bias table [row][GPS] (bf16); with a K
    // split, the chunks' partial tiles [slot][tile][chunk].
    u32x4_t* xb = lds_a4;
    u32x4_t* xh = xb + (size_t)KS * NB * 64;
    float* xs = reinterpret_cast<float*>(xh + (size_t)nkc * KSG * NB * 2 * LV);
    char* wbase0 = reinterpret_cast<char*>(xs + (size_t)KS * MT);
    char* wbase = wbase0 + (size_t)wave * affine_mfma_wave_bytes(GPS);
    // the k-block's scales [group][row]: 4- and 8-bit as fp32 (each bf16 is
    // written into the high half of a dword whose low half stays zero, so the
    // dword reads back as the exact fp32 value with no conversion), 2-bit
    // (8 groups) as bf16
    constexpr bool SB32 = GPK <= 4;
    uint16_t* sbuf = reinterpret_cast<uint16_t*>(wbase);                        // [GPK][16] bf16 / fp32
    uint16_t* btab = reinterpret_cast<uint16_t*>(wbase + 256);                  // [16][GPS]
    float* pbuf = reinterpret_cast<float*>(wbase0 + (size_t)NW * affine_mfma_wave_bytes(GPS));

    // ---- ring of D k-blocks: two whole-line loads + the block's scales and
    // biases (lane l: 4 bits: row l/4, group l%4; 2 bits: row l/4, groups
    // 2(l%4) and 2(l%4) + 1 in one 32-bit load; 8 bits: row (l/2)%16, group
    // l%2)
    u32x4_t wa[D][2];
    uint32_t sw[D], bw[D];
    int64_t f_tile = u;
    int f_b = kb_lo;
    const int h = lane & 15;
    const uint32_t voff = (uint32_t)((h & 7) * row_bytes + 16 * ((h < 8 ? 0 : 4) + c));
    // rows 8..15: the row offset goes in the vector offset, which is the
    // part of the address the buffer range check covers
    const uint32_t voff_hi = voff + (uint32_t)(8 * row_bytes);
    const uint32_t goff = BITS == 4 ? (uint32_t)(((lane >> 2) * gpr + (lane & 3)) * 2)
                        : BITS == 2 ? (uint32_t)(((lane >> 2) * gpr + 2 * (lane & 3)) * 2)
                                    : (uint32_t)((((lane >> 1) & 15) * gpr + (lane & 1)) * 2);
    auto fetch = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        const int64_t n0 = f_tile * 16;
        const int64_t rows = a.N - n0;
        const __amdgpu_buffer_rsrc_t rw = tile_rsrc(static_cast<const char*>(a.w0) + n0 * row_bytes, rows * row_bytes);
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.scales + n0 * gpr, rows * gpr * 2);
        const __amdgpu_buffer_rsrc_t rb = tile_rsrc(a.biases + n0 * gpr, rows * gpr * 2);
        if constexpr (BITS == 2) {
            sw[d] = __builtin_amdgcn_raw_buffer_load_b32(rs, goff, 2 * GPK * f_b, kLoadNT);
            bw[d] = __builtin_amdgcn_raw_buffer_load_b32(rb, goff, 2 * GPK * f_b, kLoadNT);
        } else {
            sw[d] = __builtin_amdgcn_raw_buffer_load_b16(rs, goff, 2 * GPK * f_b, kLoadNT);
            bw[d] = __builtin_amdgcn_raw_buffer_load_b16(rb, goff, 2 * GPK * f_b, kLoadNT);
        }
        wa[d][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, 128 * f_b, kLoadNT));
        wa[d][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff_hi, 128 * f_b, kLoadNT));
        const bool wrap = f_b + 1 == kb_hi;
        f_b = wrap ? kb_lo : f_b + 1;
        f_tile += wrap ? U : 0;
    };

    // XR: the row's x^T operands (k-steps 0..31) and code offsets (groups
    // 0..15) of the lane's column, from LDS once the prologue has staged them
    u32x4_t xr[XRS];
    float zr[XR ? 16 : 1];
    f32x4_t acc[NB], accb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = accb[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int c_b = kb_lo;                     // k-block being consumed
    int64_t c_tile = u;                  // its tile
    int ti = 0;                          // tiles finished (K split: partials staged)
    const bool hi8 = (lane & 8) != 0;
    uint32_t cmask = AffineMma<BITS>::MASK, cbias = 0x43004300u;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+v"(cbias));
    const u32x4_t* xhj = xh + (size_t)j * KSG * NB * 2 * LV;
    // vector stores of whole output quads: N % 4 == 0 and y addressable by a
    // 32-bit buffer offset
    const int esz = a.out_f32 ? 4 : 2;
    const bool vec_store = a.N % 4 == 0 && (int64_t)a.M * a.N * esz < 0x7FFFFFF0;
    const __amdgpu_buffer_rsrc_t ry = tile_rsrc(a.y, (int64_t)a.M * a.N * esz);
    constexpr uint32_t kDrop = 0x80000000u;
    // row argmax (a.amx, whole tiles only): the lane's running maximum of
    // its outputs of row 16b + r, per column block b
    float amx_v[NB];
    int amx_i[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        amx_v[b] = amx_neutral_value();
        amx_i[b] = kAmxNoIndex;
    }

    auto consume = [&](auto Dd) __attribute__((always_inline)) {
        constexpr int d = decltype(Dd)::value;
        // the k-block's scales and biases into the wavefront's tables (LDS
        // operations of one wavefront take effect in program order)
        {
            // raw values straight from the loads: arithmetic on them here
            // would be hoisted into the loop latch and wait there
            const int rel = GPK * (c_b - kb_lo);
            if constexpr (BITS == 4) {
                sbuf[((lane & 3) * 16 + (lane >> 2)) * 2 + 1] = (uint16_t)sw[d];
                const int ti2 = (lane >> 2) * GPS + rel + (lane & 3);
                btab[ti2] = (uint16_t)bw[d];
            } else if constexpr (BITS == 2) {
                sbuf[(2 * (lane & 3)) * 16 + (lane >> 2)] = (uint16_t)sw[d];
                sbuf[(2 * (lane & 3) + 1) * 16 + (lane >> 2)] = (uint16_t)(sw[d] >> 16);
                const int ti2 = ((lane >> 2) * GPS + rel + 2 * (lane & 3)) >> 1;   // even group: one 32-bit word
                reinterpret_cast<uint32_t*>(btab)[ti2] = bw[d];
            } else {
                // lanes 32..63 repeat lanes 0..31 (same values, same places)
                sbuf[((lane & 1) * 16 + ((lane >> 1) & 15)) * 2 + 1] = (uint16_t)sw[d];
                const int ti2 = ((lane >> 1) & 15) * GPS + rel + (lane & 1);
                btab[ti2] = (uint16_t)bw[d];
            }
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
        for (int gi = 0; gi < GPK; ++gi) {
            // scales of rows 4c .. 4c + 3, group gi
            float sc[4];
            if constexpr (SB32) {
                const float4 s4 = *reinterpret_cast<const float4*>(sbuf + (gi * 16 + 4 * c) * 2);
                sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
            } else {
                const uint2 s4 = *reinterpret_cast<const uint2*>(sbuf + gi * 16 + 4 * c);
                sc[0] = __uint_as_float(s4.x << 16); sc[1] = __uint_as_float(s4.x & 0xFFFF0000u);
                sc[2] = __uint_as_float(s4.y << 16); sc[3] = __uint_as_float(s4.y & 0xFFFF0000u);
            }
            // the group's 16 codes of this lane as the A operands of its two k-steps
            u32x4_t A0, A1, H0, H1;
            if constexpr (BITS == 4) {
                A0 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1)], cmask, cbias);
                A1 = codes4_to_bf16(pc[gi >> 1][2 * (gi & 1) + 1], cmask, cbias);
            } else if constexpr (BITS == 2) {
                A0 = codes2_to_bf16(pc[gi >> 2][gi & 3], 0, cmask, cbias);
                A1 = codes2_to_bf16(pc[gi >> 2][gi & 3], 1, cmask, cbias);
            } else {
                codes8_to_bf16(pc[gi][0], pc[gi][1], cmask, cbias, A0, H0);
                codes8_to_bf16(pc[gi][2], pc[gi][3], cmask, cbias, A1, H1);
            }
            const int S0 = 2 * (GPK * c_b + gi);
            const float* d0g = xs + (size_t)(GPK * c_b + gi) * MT + r;   // code offsets of the group's columns
            const int GX = XR ? GPK * d + gi : 0;                          // the group (XR: c_b == d)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const u32x4_t B0 = XR ? xr[2 * GX] : xb[(S0 * NB + b) * 64 + lane];
                const u32x4_t B1 = XR ? xr[2 * GX + 1] : xb[((S0 + 1) * NB + b) * 64 + lane];
                f32x4_t dg = mfma16x16x32(A0, B0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                dg = mfma16x16x32(A1, B1, dg);
                if constexpr (BITS == 8) {
                    f32x4_t dh = mfma16x16x32(H0, B0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    dh = mfma16x16x32(H1, B1, dh);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dg[i] = fmaf(16.0f, dh[i], dg[i]);
                }
                const float z = XR ? zr[GX] : d0g[16 * b];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[b][i] = fmaf(sc[i], dg[i] - z, acc[b][i]);
            }
        }
        if (++c_b == kb_hi) {
            // end of the tile (or of its K-chunk): the bias term
            c_b = kb_lo;
            const bool lv = lane < LV;
#pragma unroll
            for (int ks = 0; ks < KSG; ++ks) {
                const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
                const u32x4_t Ab = lv ? *reinterpret_cast<const u32x4_t*>(btab + r * GPS + 32 * ks + 8 * c) : z;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const u32x4_t Xh = lv ? xhj[((ks * NB + b) * 2 + 0) * LV + lane] : z;
                    const u32x4_t Xl = lv ? xhj[((ks * NB + b) * 2 + 1) * LV + lane] : z;
                    accb[b] = mfma16x16x32(Ab, Xh, accb[b]);
                    accb[b] = mfma16x16x32(Ab, Xl, accb[b]);
                }
            }
            // lane (c, r) holds rows 4c .. 4c + 3 of column 16b + r
            if (nkc == 1) {
                // whole tile: store now (staging would not coalesce either:
                // consecutive lanes write different rows of y).  Lane (c, r)
                // holds 4 consecutive outputs of row m of y: one 8- or
                // 16-byte buffer store (dropped past the end) when N % 4 == 0
                // keeps them aligned, else one store per output.
                const int64_t n0 = c_tile * 16 + 4 * c;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int m = 16 * b + r;
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = acc[b][i] + accb[b][i];
                    if (a.amx) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (m < a.M && n0 + i < a.N) amx_take(amx_v[b], amx_i[b], v[i], (int)(n0 + i));
                    } else if (vec_store) {
                        const uint32_t off = (m < a.M && n0 < a.N) ? (uint32_t)(((int64_t)m * a.N + n0) * esz) : kDrop;
                        if (a.out_f32) {
                            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                                            __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                                   ry, off, 0, 0);
                        } else {
                            const uint32_t p0 = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
                            const uint32_t p1 = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
                            __builtin_amdgcn_raw_buffer_store_b64(u32x2v_t{p0, p1}, ry, off, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if (m < a.M && n0 + i < a.N) {
                                const size_t o = (size_t)m * a.N + (size_t)(n0 + i);
                                if (a.out_f32) reinterpret_cast<float*>(a.y)[o] = v[i];
                                else reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16_rne(v[i]);
                            }
                        }
                    }
                }
            } else {
                float* pt = pbuf + ((((size_t)(wave >> lk) * a.tmax + ti) * nkc + j) * PER_TILE);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pt[(4 * c + i) * MT + 16 * b + r] = acc[b][i] + accb[b][i];
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = accb[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            c_tile += U;
            ++ti;
        }
    };

    // prologue: D k-blocks, then stage x^T (pair order within each 8-k chunk)
    // with the sums of each staged 8 x, then each chunk's group sums X as
    // bf16 high/low fragments, clear the bias table (groups past the chunk's
    // end stay zero), and the code offsets D0
    static_for<0, D>([&](auto Dd) __attribute__((always_inline)) { fetch(Dd); });
    {
        constexpr int XB = 4;
        const int ntask = KS * NB * 64;
        for (int t0 = threadIdx.x; t0 < ntask; t0 += XB * kAffineMfmaThreads) {
            u32x4_t v[XB];
            float p8[XB];
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kAffineMfmaThreads;
                const int l = t & 63;
                const int sb = t >> 6;
                const int S = sb / NB, b = sb - S * NB;
                const int m = 16 * b + (l & 15);
                v[i] = u32x4_t{0u, 0u, 0u, 0u};
                p8[i] = 0.0f;
                if (t < ntask && m < a.M) v[i] = stage_x_operand<BITS>(a.x + (size_t)m * a.K, S, l >> 4, p8[i]);
            }
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int t = t0 + i * kAffineMfmaThreads;
                if (t < ntask) {
                    xb[t] = v[i];
                    // sum of the k-step's 32 x of column m: this lane's 8,
                    // then across the four quarters (lanes 16 apart; the whole
                    // wavefront is here: ntask is a multiple of 64)
                    const int l = t & 63;
                    const int sb = t >> 6;
                    const int S = sb / NB, b = sb - S * NB;
                    const int m = 16 * b + (l & 15);
                    float q = p8[i];
                    q += __shfl_xor(q, 16);
                    q += __shfl_xor(q, 32);
                    if (l < 16) xs[S * MT + m] = q;
                }
            }
        }
        for (int t = lane; t < 8 * GPS; t += 64)           // the bias table (16 x GPS bf16) as 32-bit words
            reinterpret_cast<uint32_t*>(btab)[t] = 0u;
        if constexpr (SB32)                                 // the fp32 scales' low halves
            for (int t = lane; t < 16 * GPK; t += 64) reinterpret_cast<uint32_t*>(sbuf)[t] = 0u;
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
        const int g_lo = GPK * (jj * KBL / nkc), g_hi = GPK * ((jj + 1) * KBL / nkc);
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
    __syncthreads();   // the sums xs are read; their space takes the offsets
    // code offsets D0[g][column]: the group's MFMA chain on zero codes (every
    // A row is (128, ..., 128), so every row of the result is the same)
    {
        const u32x4_t A0 = u32x4_t{kZeroCodePair, kZeroCodePair, kZeroCodePair, kZeroCodePair};
        for (int task = wave; task < (KS / 2) * NB; task += NW) {
            const int g = task / NB, b = task - g * NB;
            const u32x4_t B0 = xb[((2 * g) * NB + b) * 64 + lane], B1 = xb[((2 * g + 1) * NB + b) * 64 + lane];
            f32x4_t d0 = mfma16x16x32(A0, B0, f32x4_t{0.f, 0.f, 0.f, 0.f});
            d0 = mfma16x16x32(A0, B1, d0);
            float z = d0[0];
            if constexpr (BITS == 8) z = fmaf(16.0f, z, z);   // the high-nibble chain is the same chain
            if (c == 0) xs[(size_t)g * MT + 16 * b + r] = z;
        }
    }
    // Every load issued so far is complete (the x loads came after the
    // weights and loads complete in order); saying so keeps a possibly
    // pending staging load out of the loop's waits.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if constexpr (XR) {
#pragma unroll
        for (int S = 0; S < XRS; ++S) xr[S] = xb[S * 64 + lane];
#pragma unroll
        for (int g = 0; g < 16; ++g) zr[g] = xs[g * MT + r];
    }
    // without a K split nothing below waits for the other wavefronts
    if (nkc == 1 && my_tiles == 0) {
        if (a.amx && lane < kArgmaxRows) amx_store(a.amx, a.amx_slots, u, lane, amx_neutral_value(), kAmxNoIndex);
        return;
    }

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
    if (nkc == 1) {
        if (a.amx) {
            // the four lane quarters hold the same rows: combine, and quarter 0
            // writes this wavefront's partials of rows 16b + r
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                amx_xor(amx_v[b], amx_i[b], 16);
                amx_xor(amx_v[b], amx_i[b], 32);
                if (c == 0) amx_store(a.amx, a.amx_slots, u, 16 * b + r, amx_v[b], amx_i[b]);
            }
            if (NB == 1 && lane >= 16 && lane < kArgmaxRows)
                amx_store(a.amx, a.amx_slots, u, lane, amx_neutral_value(), kAmxNoIndex);
        }
        return;
    }

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
// 1024 LM head at M = 16, depth 4 with one workgroup (8 wavefronts, ~64 KB
// in flight) per CU measured fastest (25.1 us; 2 workgroups 26.1 us, level
// at M = 4; 3 workgroups ~20% slower).
constexpr int kAffineMfmaDepth = 4;
constexpr int kAffineMfmaWgPerCu = 1;

// LDS bytes of one workgroup with nkc K-chunks per tile and, for nkc > 1,
// tmax tiles per slot staged as partials.
inline size_t affine_mfma_lds_bytes(int MT, int K, int bits, int nkc, int64_t tmax)
{
    const int gps = affine_mfma_gps(K, bits, nkc);
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

template <int BITS, int MT, int GPS, bool XR = false>
hipError_t launch_affine_mfma_one(const ProjArgs& a, int nkc, hipStream_t s)
{
    if (XR && (a.K != 1024 || nkc != 1)) return hipErrorInvalidValue;
    const void* fn = reinterpret_cast<const void*>(&affine_mfma_kernel<BITS, MT, kAffineMfmaDepth, GPS, XR>);
    {
        hipError_t e = raise_lds_limit(fn, kMfmaStreamLdsMax);
        if (e != hipSuccess) return e;
    }
    int cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    int bpc = kAffineMfmaWgPerCu, blocks = 0;
    int64_t tmax = 0;
    size_t lds = 0;
    for (;;) {
        affine_mfma_geometry(T, nkc, cus, bpc, blocks, tmax);
        lds = affine_mfma_lds_bytes(MT, a.K, BITS, nkc, tmax);
        if (lds > kMfmaStreamLdsMax) return hipErrorInvalidValue;
        int occ = 0;
        e = occupancy(occ, fn, kAffineMfmaThreads, lds);
        if (e != hipSuccess) return e;
        if (occ >= bpc || bpc == 1) break;
        bpc = occ < 1 ? 1 : occ;
    }
    // row argmax: one partial per wavefront, whole tiles only
    if (a.amx && (nkc != 1 || (int64_t)blocks * (kAffineMfmaThreads / 64) > a.amx_slots)) return hipErrorInvalidValue;
    if (a.amx_producers) *a.amx_producers = (int64_t)blocks * (kAffineMfmaThreads / 64);
    ProjArgs a2 = a;
    a2.tpw = 1;
    a2.tmax = tmax;
    int lk = 0;
    while ((1 << lk) < nkc) ++lk;
    a2.ksplit_log2 = lk;
    hipLaunchKernelGGL((affine_mfma_kernel<BITS, MT, kAffineMfmaDepth, GPS, XR>), dim3(blocks), dim3(kAffineMfmaThreads), lds, s, a2);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_affine_mfma_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    const int nkc = 1 << c.ksplit_log2;
    // every chunk at least one k-block
    if (nkc > kAffineMfmaThreads / 64 || nkc > affine_mfma_kbl(a.K, BITS)) return hipErrorInvalidValue;
    const bool w = c.MT == 16;
    switch (affine_mfma_gps(a.K, BITS, nkc)) {
        case 8: return w ? launch_affine_mfma_one<BITS, 16, 8>(a, nkc, s) : launch_affine_mfma_one<BITS, 32, 8>(a, nkc, s);
        case 16:
            if constexpr (BITS == 4)
                if (w && a.K == 1024 && nkc == 1) return launch_affine_mfma_one<BITS, 16, 16, true>(a, nkc, s);
            return w ? launch_affine_mfma_one<BITS, 16, 16>(a, nkc, s) : launch_affine_mfma_one<BITS, 32, 16>(a, nkc, s);
        case 32: return w ? launch_affine_mfma_one<BITS, 16, 32>(a, nkc, s) : launch_affine_mfma_one<BITS, 32, 32>(a, nkc, s);
        case 64: return w ? launch_affine_mfma_one<BITS, 16, 64>(a, nkc, s) : launch_affine_mfma_one<BITS, 32, 64>(a, nkc, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
