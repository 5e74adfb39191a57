// Persistent matrix-core kernel for affine GEMVs with codes of 2 to 8 bits
// (M padded to 16 or 32) that copies whole 16-row tiles into LDS, as the
// dense tile kernel (mfma_tile.h) does.
//
// Widths: 2, 4 and 8 bits take the operand orders of affine_mfma.h; 3, 5, 6
// and 7 bits a natural order, each lane quarter extracting its 16 codes of a
// group from a bit window (AffineTileWidth, codes_window_to_bf16).
//
// A tile is RB blocks of 16 rows of codes (16 RB K b / 8 consecutive bytes
// of HBM) plus the rows' scales and biases.  Each of the 8 wavefronts of a
// workgroup copies its share of the code bytes (1 KB per instruction, 16
// bytes per lane, straight into LDS, in address order) and the scales and
// biases of its own rows and k range (4 bytes per lane).  Every wavefront
// issues the same number of copies per tile, so the waits can count them
// exactly.
//
// The wavefronts split a tile into RB row blocks times KS = 8 / RB k chunks:
// wavefront w owns row block w / KS and k in [kc K/KS, (kc+1) K/KS) with
// kc = w % KS, i.e. K/(64 KS) groups of 64 codes, of every tile:
//   * its x^T B operands for that range stay in registers for the whole
//     launch, in the k order of the width's A operands, with the group sums
//     X_g = sum_k x_k of each of its columns;
//   * with them, the code offsets D0_g: the group's MFMA chain run on zero
//     codes (every A row (128, ..., 128)), i.e. C X_g as the matrix core
//     computes it (C = 128, or 2176 for 8 bits);
//   * per tile it turns the group scales and biases into an fp32 table
//     (s, bias) in its own LDS area;
//   * per group it reads the lane's code dwords of its row from LDS, places
//     them in bf16 mantissas (128 + q; 8-bit codes as two nibble operands),
//     runs the group's two k-steps into a fresh 16 x 16 tile D and adds
//     s (D - D0_g) + bias X_g in fp32 -- the factored form of
//     sum_k x_k (s q_k + bias); a group of zero codes gives D == D0_g bit for
//     bit and so adds exactly bias X_g.
// The KS partial blocks of a row block are summed through LDS in k-chunk
// order (fixed: results do not depend on M); each thread stores 16 RB MT /
// 512 outputs per tile with one buffer store each.  Larger RB amortizes the
// per-tile synchronization over more bytes (4-bit K = 1024 rows are only 512
// bytes).  Tiles are dealt in XCD-major order (see mfma_tile.h).
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).
#pragma once

#include "affine_mfma.h"
#include "mfma_tile.h"

namespace aqg {
namespace detail {

template <int BITS, int MT, int K, int RB, int NBUF, int NWV = kMfmaTileWaves>
struct AffineTileLayout {
    static constexpr int NT = 64 * NWV;           // threads per workgroup
    static constexpr int KS = NWV / RB;           // k chunks per row block
    static constexpr int ROWB = K * BITS / 8;     // code bytes per row
    static constexpr int CP = 16 * RB * ROWB / 1024;   // 1 KB code pieces per tile
    static constexpr int CPW = CP / NWV;
    static constexpr int CODE = CP * 1040;        // LDS: pieces with a 16-byte pad each
    static constexpr int GW = K / (64 * KS);      // groups per wavefront
    static constexpr int GPR = K / 64;            // groups per row
    static constexpr int SBW = 16 * GW * 2;       // bytes of one wavefront's scales (16 rows x GW)
    static constexpr int SBL = SBW / 4;           // lanes copying them, 4 bytes each
    static constexpr int TILE = CODE + 2 * NWV * SBW;
    static constexpr int OPT = CPW + 2;           // copies per wavefront per tile
    static constexpr int NB = MT / 16;
    static constexpr int PW = NB * 4 * 65;
    static constexpr int PART = NWV * PW * 4;
    static constexpr int NSTO = (16 * RB * MT + NT - 1) / NT;   // stores per thread per tile
    static constexpr int TAB = NWV * 2 * GW * 16 * 4;   // per-wavefront (s, bias) tables
    static constexpr int D0T = NWV * GW * NB * 16 * 4;  // per-wavefront code offsets
    static constexpr size_t LDS = (size_t)NBUF * TILE + PART + TAB + D0T;
    static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8, "row blocks divide the wavefronts");
    static_assert(K % (64 * KS) == 0, "whole groups per wavefront");
    static_assert(CP % NWV == 0 && CP > 0, "code pieces split evenly over the wavefronts");
    static_assert(NWV % RB == 0, "row blocks divide the wavefronts");
    static_assert(GW % 2 == 0 && SBL <= 64, "scales come as pairs of groups, one copy instruction per wavefront");
};

// 4 bytes per lane from buffer offset soff + voff into LDS at lds + 4 lane.
__device__ __forceinline__ void copy_dword_to_lds(u32x4v_t rs, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}

// Widths 3, 5, 6, 7: lane quarter c of a row takes codes 16c .. 16c + 15 of
// each group, and k-step h the codes 16c + 8h .. + 7, in natural order (2, 4
// and 8 bits keep the orders of affine_mfma.h).
template <int B> struct AffineTileWidth {
    static constexpr bool NATURAL = B != 2 && B != 4 && B != 8;
    static constexpr int NWN = (16 * B + 31) / 32;   // words of a lane's 16-code window
    static constexpr uint32_t MASK = (1u << B) - 1u;
};

// x^T operand of k-step S (group S / 2, half S % 2) in natural k order for
// lane quarter c: x[64 (S / 2) + 16 c + 8 (S % 2) .. + 7]; also its sum.
__device__ __forceinline__ u32x4_t stage_x_natural(const uint16_t* xr, int S, int c, float& sum)
{
    const uint4 v = *reinterpret_cast<const uint4*>(xr + 64 * (S >> 1) + 16 * c + 8 * (S & 1));
    sum = ((bf16_to_f32(v.x & 0xFFFFu) + bf16_to_f32(v.x >> 16)) + (bf16_to_f32(v.y & 0xFFFFu) + bf16_to_f32(v.y >> 16))) +
          ((bf16_to_f32(v.z & 0xFFFFu) + bf16_to_f32(v.z >> 16)) + (bf16_to_f32(v.w & 0xFFFFu) + bf16_to_f32(v.w >> 16)));
    return u32x4_t{v.x, v.y, v.z, v.w};
}

// Codes 8H .. 8H + 7 of a lane's window wn (code i at bits B i, LSB first)
// as bf16 pairs (128 + q_{2t}, 128 + q_{2t+1}), t = 0..3.  m = the B-bit
// mask, mh = m << 16, cb = 0x43004300, all opaque registers, and only plain
// C, so the compiler sees every write of these MFMA operands.
template <int B, int H>
__device__ __forceinline__ u32x4_t codes_window_to_bf16(const uint32_t (&wn)[AffineTileWidth<B>::NWN], uint32_t m,
                                                       uint32_t mh, uint32_t cb)
{
    u32x4_t o;
    static_for<0, 4>([&](auto Tc) __attribute__((always_inline)) {
        constexpr int t = decltype(Tc)::value;
        constexpr int bit = (8 * H + 2 * t) * B;
        constexpr int k = bit >> 5, sh = bit & 31;
        uint32_t w;
        if constexpr (sh + 2 * B <= 32) w = wn[k] >> sh;
        else w = __builtin_amdgcn_alignbit(wn[k + 1], wn[k], sh);
        o[t] = (w & m) | ((w << (16 - B)) & mh) | cb;
    });
    return o;
}

template <int BITS, int MT, int K, int RB, int NBUF, int NWV = kMfmaTileWaves>
__global__ void __launch_bounds__(64 * NWV) affine_tile_kernel(ProjArgs a)
{
    using L = AffineTileLayout<BITS, MT, K, RB, NBUF, NWV>;
    constexpr int KS = L::KS;
    constexpr int NB = L::NB;
    constexpr int GW = L::GW;
    using WD = AffineTileWidth<BITS>;
    static_assert(NBUF >= 2 && NBUF <= 6, "ring of 2..6 tiles");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;
    const int r = lane & 15;
    const int64_t T = ((int64_t)a.N + 16 * RB - 1) / (16 * RB);
    const int rb = wave / KS, kc = wave % KS;
    const int64_t G8 = gridDim.x / 8;
    const int64_t first = (gridDim.x % 8 == 0) ? (int64_t)(blockIdx.x % 8) * G8 + blockIdx.x / 8 : blockIdx.x;
    const int64_t stride = gridDim.x;
    if (first >= T) return;
    const int64_t ntile = (T - 1 - first) / stride + 1;

    float* part = reinterpret_cast<float*>(mfma_tile_lds<NBUF, L::PART>());
    float* tab = reinterpret_cast<float*>(mfma_tile_lds<NBUF + 1, L::TAB>()) + wave * 2 * GW * 16;   // [2][GW][16]

    // copy local tile j into buffer B: code pieces wave*CPW .. + CPW - 1, then
    // this wavefront's scales and biases ([16 rows][GW] bf16 each): lane
    // l < SBL copies groups 2 (l % (GW/2)) + {0, 1} of row 16 rb + l / (GW/2)
    const int gw0 = kc * GW;
    const uint32_t sb_voff = (uint32_t)(((16 * rb + lane / (GW / 2)) * L::GPR + gw0 + 2 * (lane % (GW / 2))) * 2);
    auto issue = [&](int64_t j, auto Bc) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
        const int64_t n0 = (first + j * stride) * 16 * RB;
        const int64_t rows = a.N - n0;
        const u32x4v_t rw = buffer_words(static_cast<const char*>(a.w0) + n0 * L::ROWB, rows * L::ROWB);
        const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)mfma_tile_lds<B, L::TILE>();
#pragma unroll
        for (int q = 0; q < L::CPW; ++q) {
            const int piece = wave * L::CPW + q;
            // the piece's offset in the vector offset, which the range check covers
            copy_1k_to_lds(rw, dst + piece * 1040, (uint32_t)(lane * 16 + piece * 1024), 0);
        }
        // only the first SBL lanes copy (a lane past a buffer's range still
        // writes zeros into LDS); lane 0 is always one of them, so each
        // wavefront issues both instructions for every tile
        const u32x4v_t rs = buffer_words(a.scales + n0 * L::GPR, rows * L::GPR * 2);
        const u32x4v_t rb = buffer_words(a.biases + n0 * L::GPR, rows * L::GPR * 2);
        if (lane < L::SBL) {
            copy_dword_to_lds(rs, dst + L::CODE + wave * L::SBW, sb_voff, 0);
            copy_dword_to_lds(rb, dst + L::CODE + (NWV + wave) * L::SBW, sb_voff, 0);
        }
    };

    // The first tile goes out before x is staged; the rest of the ring only
    // after it: the wait for x (which the compiler places as a wait for every
    // load in flight) then covers one tile rather than the whole ring, and
    // the first tile's arithmetic overlaps the others' copies (with few
    // tiles per workgroup this start is a large part of the call).
    issue(0, Int<0>{});

    // x^T operands of this wavefront's 2 GW k-steps, the group sums and the
    // groups' code offsets
    u32x4_t xr[2 * GW][NB];
    float X[GW][NB];
    // the offsets live in LDS, this wavefront's [GW][NB][16 columns]: each
    // lane stores the value of its own column and later reads back the
    // address it wrote (the four lanes of a column write the same value)
    float* d0w = reinterpret_cast<float*>(mfma_tile_lds<NBUF + 2, L::D0T>()) + wave * GW * NB * 16;
    const int kw = kc * (K / KS);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int m = 16 * b + r;
        const uint16_t* xrow = a.x + (size_t)(m < a.M ? m : 0) * K + kw;
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            float s0 = 0.f, s1 = 0.f;
            if constexpr (WD::NATURAL) {
                xr[2 * g][b] = stage_x_natural(xrow, 2 * g, c, s0);
                xr[2 * g + 1][b] = stage_x_natural(xrow, 2 * g + 1, c, s1);
            } else {
                xr[2 * g][b] = stage_x_operand<BITS>(xrow, 2 * g, c, s0);
                xr[2 * g + 1][b] = stage_x_operand<BITS>(xrow, 2 * g + 1, c, s1);
            }
            if (m >= a.M) {
                xr[2 * g][b] = xr[2 * g + 1][b] = u32x4_t{0u, 0u, 0u, 0u};
                s0 = s1 = 0.f;
            }
            // the group's sum over the four lane quarters, in a fixed order
            float v = s0 + s1;
            const float v16 = __shfl_xor(v, 16);
            const float p = (c & 1) ? v16 + v : v + v16;
            const float p32 = __shfl_xor(p, 32);
            X[g][b] = (c & 2) ? p32 + p : p + p32;
            const u32x4_t Z = u32x4_t{kZeroCodePair, kZeroCodePair, kZeroCodePair, kZeroCodePair};
            f32x4_t d0 = mfma16x16x32(Z, xr[2 * g][b], f32x4_t{0.f, 0.f, 0.f, 0.f});
            d0 = mfma16x16x32(Z, xr[2 * g + 1][b], d0);
            d0w[(g * NB + b) * 16 + r] = BITS == 8 ? fmaf(16.0f, d0[0], d0[0]) : d0[0];   // 8 bits: the high-nibble chain is the same
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    static_for<1, NBUF>([&](auto Bc) __attribute__((always_inline)) {
        if (decltype(Bc)::value < ntile) issue(decltype(Bc)::value, Bc);
    });
    barrier_only();   // tile 0 is in LDS: every wavefront waited for its copies

    uint32_t cmask = WD::NATURAL ? WD::MASK : AffineMma<BITS == 2 || BITS == 4 ? BITS : 8>::MASK;
    uint32_t cmaskh = WD::MASK << 16, cbias = 0x43004300u;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+s"(cmaskh));
    asm volatile("" : "+v"(cbias));
    // natural widths: first word and bit of the lane's 16-code window in a group
    const int lw0 = (16 * c * BITS) >> 5;
    const bool lodd = ((16 * c * BITS) & 31) != 0;

    const int t = threadIdx.x;
    const int esz = a.out_f32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ry = tile_rsrc(a.y, (int64_t)a.M * a.N * esz);
    constexpr uint32_t kDrop = 0x80000000u;

    auto step = [&](int64_t j, auto Bc) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
        const char* tb = mfma_tile_lds<B, L::TILE>();
        // (s, bias) of this wavefront's groups, rows 0..15: lane e < 16 GW
        // takes row e % 16 of group e / 16
#pragma unroll
        for (int e0 = 0; e0 < 16 * GW; e0 += 64) {
            const int e = e0 + lane;
            if (e < 16 * GW) {
                const int row = e & 15, g = e >> 4;
                const uint16_t* sp = reinterpret_cast<const uint16_t*>(tb + L::CODE + wave * L::SBW);
                const uint16_t* bp = reinterpret_cast<const uint16_t*>(tb + L::CODE + (NWV + wave) * L::SBW);
                const float s = bf16_to_f32(sp[row * GW + g]);
                const float bi = bf16_to_f32(bp[row * GW + g]);
                tab[g * 16 + row] = s;
                tab[(GW + g) * 16 + row] = bi;
            }
        }
        f32x4_t acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // row r's codes: byte offset of group g0 + g within the tile
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            const int off = (16 * rb + r) * L::ROWB + (gw0 + g) * 8 * BITS;   // group start
            // 2, 4, 8 bits: a group never straddles a 1 KB piece
            const char* gp = tb + (off >> 10) * 1040 + (off & 1023) + 4 * c;
            u32x4_t A0, A1, H0, H1;
            if constexpr (WD::NATURAL) {
                // the window's words (each placed by its own piece: odd-width
                // groups can straddle pieces), shifted by 16 bits when the
                // window starts mid-word
                uint32_t raw[WD::NWN + 1], wn[WD::NWN];
#pragma unroll
                for (int k = 0; k <= WD::NWN; ++k) {
                    const int ab = off + 4 * (lw0 + k);
                    raw[k] = *reinterpret_cast<const uint32_t*>(tb + (ab >> 10) * 1040 + (ab & 1023));
                }
#pragma unroll
                for (int k = 0; k < WD::NWN; ++k) wn[k] = lodd ? __builtin_amdgcn_alignbit(raw[k + 1], raw[k], 16) : raw[k];
                A0 = codes_window_to_bf16<BITS, 0>(wn, cmask, cmaskh, cbias);
                A1 = codes_window_to_bf16<BITS, 1>(wn, cmask, cmaskh, cbias);
            } else if constexpr (BITS == 4) {
                A0 = codes4_to_bf16(*reinterpret_cast<const uint32_t*>(gp), cmask, cbias);
                A1 = codes4_to_bf16(*reinterpret_cast<const uint32_t*>(gp + 16), cmask, cbias);
            } else if constexpr (BITS == 2) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(gp);
                A0 = codes2_to_bf16(w, 0, cmask, cbias);
                A1 = codes2_to_bf16(w, 1, cmask, cbias);
            } else {
                codes8_to_bf16(*reinterpret_cast<const uint32_t*>(gp), *reinterpret_cast<const uint32_t*>(gp + 16),
                               cmask, cbias, A0, H0);
                codes8_to_bf16(*reinterpret_cast<const uint32_t*>(gp + 32), *reinterpret_cast<const uint32_t*>(gp + 48),
                               cmask, cbias, A1, H1);
            }
            const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(tab + g * 16 + 4 * c);
            const f32x4_t cc = *reinterpret_cast<const f32x4_t*>(tab + (GW + g) * 16 + 4 * c);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4_t dg = mfma16x16x32(A0, xr[2 * g][b], f32x4_t{0.f, 0.f, 0.f, 0.f});
                dg = mfma16x16x32(A1, xr[2 * g + 1][b], dg);
                if constexpr (BITS == 8) {
                    f32x4_t dh = mfma16x16x32(H0, xr[2 * g][b], f32x4_t{0.f, 0.f, 0.f, 0.f});
                    dh = mfma16x16x32(H1, xr[2 * g + 1][b], dh);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dg[i] = fmaf(16.0f, dh[i], dg[i]);
                }
                const float z0 = d0w[(g * NB + b) * 16 + r];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[b][i] = fmaf(sc[i], dg[i] - z0, fmaf(cc[i], X[g][b], acc[b][i]));
            }
        }
        float* pw = part + wave * L::PW;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[(b * 4 + i) * 65 + lane] = acc[b][i];
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
        barrier_only();

        // every wavefront is done with buffer B: refill it with tile j + NBUF
        if (j + NBUF < ntile) issue(j + NBUF, Bc);

        // output o = t + 512 u of the tile: column m = o / (16 RB), row
        // 16 rb' + n16 with o % (16 RB) = 16 rb' + n16 (consecutive threads,
        // consecutive rows of one column)
#pragma unroll
        for (int u = 0; u < L::NSTO; ++u) {
            const int o = t + L::NT * u;
            const bool valid = o < 16 * RB * MT;
            const int om = valid ? o / (16 * RB) : 0, nl = o % (16 * RB);
            const int rbo = nl >> 4, n16 = nl & 15;
            const float* p = part + (rbo * KS) * L::PW + ((om >> 4) * 4 + (n16 & 3)) * 65 + (n16 >> 2) * 16 + (om & 15);
            float v = p[0];
#pragma unroll
            for (int k2 = 1; k2 < KS; ++k2) v += p[k2 * L::PW];
            const int64_t n = (first + j * stride) * 16 * RB + nl;
            const uint32_t off = (valid && om < a.M && n < a.N) ? (uint32_t)(((int64_t)om * a.N + n) * esz) : kDrop;
            if (a.out_f32) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), ry, off, 0, 0);
        }

        // Tile j + 1 must be in LDS before the next step (see mfma_tile.h).
        // Issued by step j + 1 - NBUF: after its copies came that step's NSTO
        // stores and, per step since, one tile's OPT copies (if the tile
        // exists) and NSTO stores.  Issued in the prologue (j = B < NBUF - 1):
        // after its copies came the prologue's later tiles and, per step 0..B,
        // one tile's copies (if it exists) and NSTO stores.
        const bool from_step = j + 1 >= NBUF;
        if (from_step) {
            const int64_t nd64 = ntile - 2 - j;
            const int nd = nd64 < 0 ? 0 : (nd64 > NBUF - 1 ? NBUF - 1 : (int)nd64);
            static_for<0, NBUF>([&](auto Dc) __attribute__((always_inline)) {
                constexpr int D = decltype(Dc)::value;
                if (nd == D) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(D * L::OPT + NBUF * L::NSTO));
            });
        } else {
            const int64_t lim = ntile < NBUF ? ntile : NBUF;
            const int64_t np = lim - (B + 2) > 0 ? lim - (B + 2) : 0;                    // later prologue tiles
            const int64_t ns = ntile - NBUF > 0 ? (ntile - NBUF < B + 1 ? ntile - NBUF : B + 1) : 0;   // tiles issued by steps 0..B
            const int q = (int)(np + ns);
            static_for<0, NBUF>([&](auto Qc) __attribute__((always_inline)) {
                constexpr int Q = decltype(Qc)::value;
                if (q == Q) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(Q * L::OPT + (B + 1) * L::NSTO));
            });
        }
        barrier_only();
    };

    for (int64_t j0 = 0; j0 < ntile; j0 += NBUF) {
        static_for<0, NBUF>([&](auto Bc) __attribute__((always_inline)) {
            const int64_t j = j0 + decltype(Bc)::value;
            if (j < ntile) step(j, Bc);
        });
    }
}

// Ring depth for (bits, K) with 16-row tiles: about 40-100 KB of tiles in
// flight, within one CU's LDS at M = 32 (8-bit K = 4096: M <= 16 only);
// 0 = shape not served.  4-bit K = 4096 keeps 2 tiles (72 KB): 3 measured
// 13% slower on 14336 x 4096 at M = 8 and 16, where a workgroup has only 3-4
// tiles; 2-bit K = 4096 keeps 3 (2 measured 10% slower).  4-bit K = 1024 is left to the other kernels: its
// tiles are 9 KB, and each group's chain (LDS read, code placement, two
// dependent MFMAs, the fp32 terms) is too short of bytes to keep the copies
// streaming with 8 wavefronts per CU (measured 38-40 us on the 151936 x 1024
// LM head against 16-29 us; 31-42 us with 64-row tiles).
inline int affine_tile_nbuf(int bits, int K, int MT)
{
    if (bits == 4 && K == 2048) return 3;
    if (bits == 4 && K == 4096) return 2;
    if (bits == 2 && K == 2048) return 5;
    if (bits == 2 && K == 4096) return 3;
    if (bits == 8 && K == 1024) return 3;
    if (bits == 8 && K == 2048) return 2;
    if (bits == 8 && K == 4096 && MT == 16) return 2;
    if (bits == 3 && K == 4096) return 3;
    if ((bits == 5 || bits == 6 || bits == 7) && K == 4096) return 2;
    if (bits == 6 && K == 2048) return 3;
    return 0;
}

template <int BITS, int MT, int K, int RB, int NBUF, int NWV = kMfmaTileWaves>
hipError_t launch_affine_tile_one(const ProjArgs& a, hipStream_t s)
{
    static_assert(AffineTileLayout<BITS, MT, K, RB, NBUF, NWV>::LDS <= 160 * 1024, "fits one CU's LDS");
    const void* fn = reinterpret_cast<const void*>(&affine_tile_kernel<BITS, MT, K, RB, NBUF, NWV>);
    int cus = 0, bpc = 0;
    hipError_t e = device_cus(cus);
    if (e == hipSuccess) e = occupancy(bpc, fn, 64 * NWV, 0);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const int64_t T = ((int64_t)a.N + 16 * RB - 1) / (16 * RB);
    int64_t blocks = (int64_t)bpc * cus;
    if (blocks > T) blocks = T;
    hipLaunchKernelGGL((affine_tile_kernel<BITS, MT, K, RB, NBUF, NWV>), dim3((unsigned)blocks), dim3(64 * NWV), 0, s, a);
    return hipGetLastError();
}

// Outputs addressable by one 32-bit buffer offset at any M (32 N 4 bytes
// below 2 GB); depends on (bits, N, K) and the column bucket only.
inline bool affine_tile_supported(int bits, int N, int K, int MT)
{
    return affine_tile_nbuf(bits, K, MT) != 0 && (int64_t)32 * N * 4 < 0x7FFFFFF0;
}

template <int BITS, int MT>
hipError_t launch_affine_tile_mt(const ProjArgs& a, hipStream_t s)
{
    if constexpr (BITS == 4) {
        switch (a.K) {
            case 2048: return launch_affine_tile_one<4, MT, 2048, 1, 3>(a, s);
            case 4096: return launch_affine_tile_one<4, MT, 4096, 1, 2>(a, s);
            default: return hipErrorInvalidValue;
        }
    } else if constexpr (BITS == 2) {
        switch (a.K) {
            case 2048: return launch_affine_tile_one<2, MT, 2048, 1, 5>(a, s);
            case 4096: return launch_affine_tile_one<2, MT, 4096, 1, 3>(a, s);
            default: return hipErrorInvalidValue;
        }
    } else if constexpr (BITS == 3) {
        return a.K == 4096 ? launch_affine_tile_one<3, MT, 4096, 1, 3>(a, s) : hipErrorInvalidValue;
    } else if constexpr (BITS == 5 || BITS == 7) {
        return a.K == 4096 ? launch_affine_tile_one<BITS, MT, 4096, 1, 2>(a, s) : hipErrorInvalidValue;
    } else if constexpr (BITS == 6) {
        switch (a.K) {
            case 2048: return launch_affine_tile_one<6, MT, 2048, 1, 3>(a, s);
            case 4096: return launch_affine_tile_one<6, MT, 4096, 1, 2>(a, s);
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.K) {
            case 1024: return launch_affine_tile_one<8, MT, 1024, 1, 3>(a, s);
            case 2048: return launch_affine_tile_one<8, MT, 2048, 1, 2>(a, s);
            case 4096:
                if constexpr (MT == 16) return launch_affine_tile_one<8, 16, 4096, 1, 2>(a, s);
                else return hipErrorInvalidValue;
            default: return hipErrorInvalidValue;
        }
    }
}

template <int BITS>
hipError_t launch_affine_tile_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (!affine_tile_supported(BITS, a.N, a.K, c.MT)) return hipErrorInvalidValue;
    switch (c.MT) {
        case 16: return launch_affine_tile_mt<BITS, 16>(a, s);
        case 32: return launch_affine_tile_mt<BITS, 32>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
