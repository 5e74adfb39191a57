// Matrix-core kernel for affine GEMVs with 2- to 8-bit codes on small
// matrices (few 16-row tiles) at M = 5..32 on gfx950: one workgroup per
// 16-row tile and block of at most 16 columns, the row's groups split over up
// to 16 wavefronts (2, 4, 8 bits: in whole 128-byte k-blocks; 3, 5, 6, 7
// bits: 2, 4 or 8 groups per wavefront).
//
// The matrices this serves are a few MB: latency-bound, so what matters is
// how soon every CU has its loads in flight (as for the dense kernel in
// mfma_split.h).  Each wavefront issues at once the codes of its KPW k-blocks
// (two whole-line loads per k-block for rows 0..7 and 8..15, the row_ror:8
// DPP select and the 4 x 4 lane-row transpose of affine_mfma.h), the scales
// and biases of its groups for the four rows its accumulator lanes own, and
// the x^T operands of its k-steps straight from global memory in the k order
// of the codes (no LDS staging, no barrier before the arithmetic).  Per group
// two MFMA k-steps on the codes placed as bf16 (128 + q; 8-bit codes as two
// nibble chains, the high one weighted 16) give D = sum_k (C + q_k) x_k, and
// (odd widths and 6 bits: each lane reads the words holding its 16-code
// window of each group, lane quarter c taking codes 16c .. 16c + 15 in
// natural k order, as affine_tile.h places them), and
// the group adds scale * (D - D0) + bias * X with X = sum_k x_k, in fp32: the
// factored form of sum_k x_k (scale * q_k + bias).  D0 is the same MFMA chain
// on zero codes (C X as the matrix core computes it), formed once per group
// from the x^T operands, so a group of zero codes adds exactly bias * X.  The partial
// 16 x 16 tiles of the wavefronts are summed through LDS in wavefront order,
// so results are deterministic and the same for every M the kernel serves.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).  Shapes: the
// decoder projections of a ~0.8B model (K = 1024 / 3584) and 4096-wide
// layers at decode batch sizes.
#pragma once
#include "affine_mfma.h"
#include "affine_tile.h"

namespace aqg {
namespace detail {

constexpr int kAffineSplitMaxWaves = 16;
// With two weight streams (the fused SwiGLU) a wavefront holds twice the
// codes, scales and biases: at most 8 wavefronts, so each may take 256
// registers.
template <int S> constexpr int affine_split_max_waves() { return S == 2 ? 8 : kAffineSplitMaxWaves; }

// Widths read as per-lane code windows (no whole-line layout) and their
// groups per unit of the KPW parameter (2, 4, 8 bits: a 128-byte k-block).
template <int BITS> constexpr bool affine_split_natural() { return !(BITS == 2 || BITS == 4 || BITS == 8); }
template <int BITS> constexpr int affine_split_gpk()
{
    if constexpr (affine_split_natural<BITS>()) return 1;
    else return AffineMma<BITS>::GPK;
}

// NDW consecutive dwords at byte offset off of a buffer (16-, 8- and 4-byte
// loads).
template <int NDW>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t (&o)[NDW])
{
    static_for<0, NDW / 4>([&](auto Qc) __attribute__((always_inline)) {
        constexpr int q = decltype(Qc)::value;
        const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * q, 0, kLoadNT));
        o[4 * q] = v[0]; o[4 * q + 1] = v[1]; o[4 * q + 2] = v[2]; o[4 * q + 3] = v[3];
    });
    constexpr int d0 = NDW / 4 * 4;
    if constexpr (NDW - d0 >= 2) {
        const u32x2v_t v = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 4 * d0, 0, kLoadNT));
        o[d0] = v[0]; o[d0 + 1] = v[1];
    }
    if constexpr ((NDW - d0) % 2 == 1)
        o[NDW - 1] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * (NDW - 1), 0, kLoadNT);
}

// CW > 0: workgroup b takes column block (b / 8) % 2 (columns [CW, 2 CW) for
// block 1) of row tile 8 (b / 16) + b % 8, so the two column blocks of a tile
// run on one XCD (workgroup b runs on XCD b % 8) and the second read of the
// tile's codes finds them in that XCD's L2.  An output's chain of MFMAs and
// fp32 operations does not depend on its column, so results are those of
// the unsplit kernel.
// S = 2: the fused SwiGLU over affine gate (w0, scales, biases) and up (w1,
// scales1, biases1) matrices: both streams of a tile through the same x^T
// operands and code offsets, two partial tiles per wavefront, and
// silu(g) * u in fp32 at the end.
// SEG: a multi-projection launch (the tile's projection looked up in the
// table at entry); a separate instantiation, so single projections load no
// table before their first weight loads.
template <int BITS, int KPW, int CW = 0, int S = 1, bool SEG = false>
__global__ void __launch_bounds__(64 * affine_split_max_waves<S>()) affine_split_kernel(ProjArgs a)
{
    extern __shared__ float lds_red[];
    constexpr bool NAT = affine_split_natural<BITS>();
    constexpr int GPK = affine_split_gpk<BITS>();  // groups per unit of KPW
    constexpr int GPW = KPW * GPK;                // groups per wavefront
    constexpr int SDW = GPW / 2;                  // dwords of one row's scales (or biases) per wavefront
    static_assert(GPW % 2 == 0, "groups come in pairs");

    int64_t tile = blockIdx.x;
    if constexpr (CW > 0) {
        static_assert(CW <= 16, "column blocks of a 16-column kernel");
        tile = (int64_t)(blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
        if (tile * 16 >= a.N) return;            // whole workgroup, before any barrier
    }
    // this tile's matrix, scales, biases, output and row count: those of its
    // projection in a multi-projection launch (locals: the kernel never
    // writes its argument block)
    SegView sv{a.w0, a.scales, a.biases, a.y, a.N, tile * 16};
    if constexpr (SEG) sv = seg_view(a, tile * 16);
    const int64_t n0 = sv.n0;
    const int N_ = sv.N;
    const void* const w0_ = sv.w;
    const uint16_t* const sc_ = sv.sc;
    const uint16_t* const bi_ = sv.bi;
    const uint16_t* x_ = a.x;
    void* y_ = sv.y;
    int M_ = a.M;
    if constexpr (CW > 0) {
        if ((blockIdx.x >> 3) & 1) {
            x_ += (size_t)CW * a.K;
            y_ = static_cast<char*>(y_) + (size_t)CW * N_ * (a.out_f32 ? 4 : 2);
            M_ -= CW;
        } else if (M_ > CW) {
            M_ = CW;
        }
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nks = blockDim.x >> 6;
    const int c = lane >> 4;
    const int r = lane & 15;
    const int64_t row_bytes = (int64_t)a.K * BITS / 8;
    const int gpr = a.K / 64;
    const int kb0 = wave * KPW;                  // first k-block of this wavefront (odd widths: group)
    const int g0 = kb0 * GPK;                    // its first group

    // codes (2, 4, 8 bits): k-block p as two whole-line loads (rows 0..7
    // and 8..15); (other widths) each group's words holding lane quarter c's
    // window of row r: NWN words from word (16 b c) / 32 of the group, the
    // window starting at bit 0 or 16 of the first
    constexpr int NWN = AffineTileWidth<BITS>::NWN;
    const uint32_t voff = NAT ? (uint32_t)(r * row_bytes + 4 * ((16 * BITS * c) >> 5))
                              : (uint32_t)((r & 7) * row_bytes + 16 * ((r < 8 ? 0 : 4) + c));
    // rows 8..15: the row offset goes in the vector offset, which is the
    // part of the address the buffer range check covers
    const uint32_t voff_hi = voff + (uint32_t)(8 * row_bytes);
    u32x4_t wa[S][NAT ? 1 : KPW][2];
    uint32_t wn[S][NAT ? GPW : 1][NWN];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const __amdgpu_buffer_rsrc_t rw =
            tile_rsrc(static_cast<const char*>(s == 0 ? w0_ : a.w1) + n0 * row_bytes, (N_ - n0) * row_bytes);
        if constexpr (NAT) {
#pragma unroll
            for (int g = 0; g < GPW; ++g)
#pragma unroll
                for (int q = 0; q < NWN; ++q)
                    wn[s][g][q] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff + 4 * q, (g0 + g) * 8 * BITS, kLoadNT);
        } else {
#pragma unroll
            for (int p = 0; p < KPW; ++p) {
                const int koff = 128 * (kb0 + p);
                wa[s][p][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, koff, kLoadNT));
                wa[s][p][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff_hi, koff, kLoadNT));
            }
        }
    }
    // scales and biases of groups g0 .. g0 + GPW - 1 for rows 4c .. 4c + 3
    // (the rows of this lane's accumulators); rows past N read as zero
    uint32_t sw[S][4][SDW], bw[S][4][SDW];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc((s == 0 ? sc_ : a.scales1) + n0 * gpr, (N_ - n0) * gpr * 2);
        const __amdgpu_buffer_rsrc_t rb = tile_rsrc((s == 0 ? bi_ : a.biases1) + n0 * gpr, (N_ - n0) * gpr * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = (uint32_t)(((4 * c + i) * gpr + g0) * 2);
            load_dwords<SDW>(rs, off, sw[s][i]);
            load_dwords<SDW>(rb, off, bw[s][i]);
        }
    }
    // x^T: lane (c, column r) holds the operands of k-steps 2g, 2g + 1 of its
    // groups, the groups' sums over all four lane quarters (fixed order) and
    // their code offsets D0 (the group's MFMA chain on zero codes)
    u32x4_t xb[2 * GPW];
    float X[GPW];
    // D0 lives in LDS (this wavefront's [GPW][16 columns] after the reduction
    // area): each lane stores the value of its own column and later reads back
    // the address it wrote (the four lanes of a column write the same value)
    float* d0w = lds_red + (size_t)S * nks * 4 * 65 + (size_t)wave * GPW * 16;
    {
        const bool have = r < M_;
        const uint16_t* xrow = x_ + (size_t)(have ? r : 0) * a.K + 64 * g0;
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            float s0 = 0.f, s1 = 0.f;
            if constexpr (NAT) {
                xb[2 * g] = stage_x_natural(xrow, 2 * g, c, s0);
                xb[2 * g + 1] = stage_x_natural(xrow, 2 * g + 1, c, s1);
            } else {
                xb[2 * g] = stage_x_operand<BITS>(xrow, 2 * g, c, s0);
                xb[2 * g + 1] = stage_x_operand<BITS>(xrow, 2 * g + 1, c, s1);
            }
            if (!have) {
                xb[2 * g] = xb[2 * g + 1] = u32x4_t{0u, 0u, 0u, 0u};
                s0 = s1 = 0.f;
            }
            const float v = s0 + s1;
            const float v16 = __shfl_xor(v, 16);
            const float p = (c & 1) ? v16 + v : v + v16;
            const float p32 = __shfl_xor(p, 32);
            X[g] = (c & 2) ? p32 + p : p + p32;
            const u32x4_t Z = u32x4_t{kZeroCodePair, kZeroCodePair, kZeroCodePair, kZeroCodePair};
            f32x4_t d0 = mfma16x16x32(Z, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
            d0 = mfma16x16x32(Z, xb[2 * g + 1], d0);
            d0w[g * 16 + r] = BITS == 8 ? fmaf(16.0f, d0[0], d0[0]) : d0[0];   // 8 bits: the high-nibble chain is the same
        }
    }

    uint32_t cmask = NAT ? AffineTileWidth<BITS>::MASK : AffineMma<NAT ? 4 : BITS>::MASK, cbias = 0x43004300u;
    uint32_t cmaskh = AffineTileWidth<BITS>::MASK << 16;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+s"(cmaskh));
    asm volatile("" : "+v"(cbias));
    const uint32_t wsh = (uint32_t)((16 * BITS * c) & 31);   // odd widths: 0 or 16
    const bool hi8 = (lane & 8) != 0;
    f32x4_t acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KPW; ++p)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        // pc[0][t]: codes of k-step t of the block, pc[1][t]: k-step 4 + t
        uint32_t pc[2][4];
        if constexpr (!NAT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t l0 = wa[s][p][0][i], l1 = wa[s][p][1][i];
                const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0, 0x128, 0xF, 0xF, false);
                const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1, 0x128, 0xF, 0xF, false);
                pc[0][i] = hi8 ? r1 : l0;
                pc[1][i] = hi8 ? l1 : r0;
            }
            transpose4x4_rows(pc[0]);
            transpose4x4_rows(pc[1]);
        }
#pragma unroll
        for (int gi = 0; gi < GPK; ++gi) {
            const int g = p * GPK + gi;          // group within the wavefront's range
            u32x4_t A0, A1, H0, H1;
            if constexpr (NAT) {
                // the window normalised to start at bit 0 (only the low 16
                // bits of the last word belong to it when it starts at 16)
                uint32_t w[NWN];
#pragma unroll
                for (int q = 0; q + 1 < NWN; ++q) w[q] = __builtin_amdgcn_alignbit(wn[s][g][q + 1], wn[s][g][q], wsh);
                w[NWN - 1] = wn[s][g][NWN - 1] >> wsh;
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
            const float z0 = d0w[g * 16 + r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sh = sw[s][i][g >> 1], bh = bw[s][i][g >> 1];
                const float sc = __uint_as_float((g & 1) ? (sh & 0xFFFF0000u) : (sh << 16));
                const float bi = __uint_as_float((g & 1) ? (bh & 0xFFFF0000u) : (bh << 16));
                acc[s][i] = fmaf(sc, dg[i] - z0, fmaf(bi, X[g], acc[s][i]));
            }
        }
    }

    // fixed-order sum of the k-splits: every wavefront stores its partial
    // tile (rows of 65 floats: conflict-free reads below), then every thread
    // adds one output's partials in order 0, 1, ..., nks-1 and stores it
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_red[(size_t)((s * nks + wave) * 4 + i) * 65 + lane] = acc[s][i];
    __syncthreads();
    // output (m, n0 + n16) lives in lane (n16 / 4) * 16 + m, element n16 % 4
    for (int o = threadIdx.x; o < 256; o += blockDim.x) {
        const int m = o >> 4, n16 = o & 15;
        const int j0 = (n16 & 3) * 65 + (n16 >> 2) * 16 + m;
        float v = lds_red[j0];
        for (int w = 1; w < nks; ++w) v += lds_red[(size_t)(w * 4) * 65 + j0];
        if constexpr (S == 2) {
            const float* pu = lds_red + (size_t)nks * 4 * 65 + j0;
            float u = pu[0];
            for (int w = 1; w < nks; ++w) u += pu[(size_t)(w * 4) * 65];
            v = (v / (1.0f + __expf(-v))) * u;
        }
        const int64_t n = n0 + n16;
        if (m >= M_ || n >= N_) continue;
        const size_t oi = (size_t)m * N_ + n;
        if (a.out_f32) reinterpret_cast<float*>(y_)[oi] = v;
        else reinterpret_cast<uint16_t*>(y_)[oi] = f32_to_bf16_rne(v);
    }
}

// k-blocks per wavefront: the smallest of 1, 2, 4 that splits the row's
// 128-byte k-blocks over at most 16 wavefronts, with at most 8 groups per
// wavefront (their x^T operands take 8 registers each; 0 if none fits).
// Widths 3, 5, 6, 7: groups per wavefront, the smallest of 2, 4, 8 that
// splits the row's groups evenly over at most max_waves wavefronts, with at
// most 64 groups in the workgroup (more windows than that do not fit the
// registers of 16 wavefronts; 0 if none).
inline int affine_split_kpw(int bits, int K, int max_waves = kAffineSplitMaxWaves)
{
    if (bits < 2 || bits > 8 || K % 64 != 0) return 0;
    if (!(bits == 2 || bits == 4 || bits == 8)) {
        const int G = K / 64;
        for (int gpw : {2, 4, 8})
            if (G % gpw == 0 && G / gpw <= max_waves && gpw * max_waves <= 64) return gpw;
        return 0;
    }
    if ((K * bits) % 1024 != 0) return 0;
    const int kbl = K * bits / 1024;
    for (int kpw : {1, 2, 4})
        if (kbl % kpw == 0 && kbl / kpw <= max_waves) return kpw * (16 / bits) <= 8 ? kpw : 0;
    return 0;
}

template <int BITS, int KPW, int S, bool SEG>
hipError_t launch_affine_split_seg(const ProjArgs& a, hipStream_t s)
{
    if (a.M > 32) return hipErrorInvalidValue;
    const int nks = affine_split_natural<BITS>() ? (a.K / 64) / KPW : (a.K * BITS / 1024) / KPW;
    const int64_t tiles = ((int64_t)a.N + 15) / 16;
    // partial tiles for the reduction (per stream), then each wavefront's code offsets
    const size_t lds = (size_t)S * nks * 4 * 65 * 4 + (size_t)nks * KPW * affine_split_gpk<BITS>() * 16 * 4;
    // M = 17..32 runs once per 16-column block, and with at most half as many
    // row tiles as CUs M = 9..16 once per 8-column block (the two blocks of a
    // tile on one XCD).
    if (a.M > 16) {
        const int64_t blocks = (tiles + 7) / 8 * 16;
        hipLaunchKernelGGL((affine_split_kernel<BITS, KPW, 16, S, SEG>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
        return hipGetLastError();
    }
    if (a.M > 8) {
        int cus = 0;
        hipError_t e = device_cus(cus);
        if (e != hipSuccess) return e;
        if (2 * tiles <= cus) {
            const int64_t blocks = (tiles + 7) / 8 * 16;
            hipLaunchKernelGGL((affine_split_kernel<BITS, KPW, 8, S, SEG>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((affine_split_kernel<BITS, KPW, 0, S, SEG>), dim3((unsigned)tiles), dim3(64 * nks), lds, s, a);
    return hipGetLastError();
}

template <int BITS, int KPW, int S>
hipError_t launch_affine_split_one(const ProjArgs& a, hipStream_t s)
{
    if constexpr (S == 1) {
        if (a.nseg > 1) return launch_affine_split_seg<BITS, KPW, S, true>(a, s);
    }
    return launch_affine_split_seg<BITS, KPW, S, false>(a, s);
}

template <int BITS, int S>
hipError_t launch_affine_split_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    (void)c;
    constexpr int GPK = affine_split_gpk<BITS>();
    if constexpr (affine_split_natural<BITS>()) {
        switch (affine_split_kpw(BITS, a.K, affine_split_max_waves<S>())) {
            case 2: return launch_affine_split_one<BITS, 2, S>(a, s);
            case 4: return launch_affine_split_one<BITS, 4, S>(a, s);
            case 8:
                if constexpr (S == 2) return launch_affine_split_one<BITS, 8, S>(a, s);
                else return hipErrorInvalidValue;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (affine_split_kpw(BITS, a.K, affine_split_max_waves<S>())) {
            case 1: return launch_affine_split_one<BITS, 1, S>(a, s);
            case 2:
                if constexpr (2 * GPK <= 8) return launch_affine_split_one<BITS, 2, S>(a, s);
                else return hipErrorInvalidValue;
            case 4:
                if constexpr (4 * GPK <= 8) return launch_affine_split_one<BITS, 4, S>(a, s);
                else return hipErrorInvalidValue;
            default: return hipErrorInvalidValue;
        }
    }
}

}  // namespace detail
}  // namespace aqg
