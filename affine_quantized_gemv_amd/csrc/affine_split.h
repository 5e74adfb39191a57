// Matrix-core kernel for affine GEMVs with 2-, 4- and 8-bit codes on small
// matrices (few 16-row tiles) at M = 5..32 on gfx950: one workgroup per
// 16-row tile and block of at most 16 columns, the row's 128-byte k-blocks
// split over up to 16 wavefronts.
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
// the group adds scale * D + (bias - C * scale) * X with X = sum_k x_k, in
// fp32: the factored form of sum_k x_k (scale * q_k + bias).  The partial
// 16 x 16 tiles of the wavefronts are summed through LDS in wavefront order,
// so results are deterministic and the same for every M the kernel serves.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64).  Shapes: the
// decoder projections of a ~0.8B model (K = 1024 / 3584) and 4096-wide
// layers at decode batch sizes.
#pragma once
#include "affine_mfma.h"

namespace aqg {
namespace detail {

constexpr int kAffineSplitMaxWaves = 16;

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
template <int BITS, int KPW, int CW = 0>
__global__ void __launch_bounds__(64 * kAffineSplitMaxWaves) affine_split_kernel(ProjArgs a)
{
    extern __shared__ float lds_red[];
    constexpr int GPK = AffineMma<BITS>::GPK;     // groups per 128-byte k-block
    constexpr int GPW = KPW * GPK;                // groups per wavefront
    constexpr float OFF = AffineMma<BITS>::OFF;
    constexpr int SDW = GPW / 2;                  // dwords of one row's scales (or biases) per wavefront
    static_assert(GPW % 2 == 0, "groups come in pairs");

    int64_t tile = blockIdx.x;
    if constexpr (CW > 0) {
        static_assert(CW <= 16, "column blocks of a 16-column kernel");
        const int b = blockIdx.x;
        tile = (int64_t)(b >> 4) * 8 + (b & 7);
        if (tile * 16 >= a.N) return;            // whole workgroup, before any barrier
        if ((b >> 3) & 1) {
            a.x += (size_t)CW * a.K;
            a.y = static_cast<char*>(a.y) + (size_t)CW * a.N * (a.out_f32 ? 4 : 2);
            a.M -= CW;
        } else if (a.M > CW) {
            a.M = CW;
        }
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nks = blockDim.x >> 6;
    const int c = lane >> 4;
    const int r = lane & 15;
    const int64_t row_bytes = (int64_t)a.K * BITS / 8;
    const int gpr = a.K / 64;
    const int64_t n0 = tile * 16;
    const int kb0 = wave * KPW;                  // first k-block of this wavefront
    const int g0 = kb0 * GPK;                    // its first group

    // codes: k-block p as two whole-line loads (rows 0..7 and 8..15)
    const uint32_t voff = (uint32_t)((r & 7) * row_bytes + 16 * ((r < 8 ? 0 : 4) + c));
    const int half_off = (int)(8 * row_bytes);
    const __amdgpu_buffer_rsrc_t rw = tile_rsrc(static_cast<const char*>(a.w0) + n0 * row_bytes, (a.N - n0) * row_bytes);
    u32x4_t wa[KPW][2];
#pragma unroll
    for (int p = 0; p < KPW; ++p) {
        const int koff = 128 * (kb0 + p);
        wa[p][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, koff, kLoadNT));
        wa[p][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, voff, koff + half_off, kLoadNT));
    }
    // scales and biases of groups g0 .. g0 + GPW - 1 for rows 4c .. 4c + 3
    // (the rows of this lane's accumulators); rows past N read as zero
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.scales + n0 * gpr, (a.N - n0) * gpr * 2);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc(a.biases + n0 * gpr, (a.N - n0) * gpr * 2);
    uint32_t sw[4][SDW], bw[4][SDW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)(((4 * c + i) * gpr + g0) * 2);
        load_dwords<SDW>(rs, off, sw[i]);
        load_dwords<SDW>(rb, off, bw[i]);
    }
    // x^T: lane (c, column r) holds the operands of k-steps 2g, 2g + 1 of its
    // groups and the groups' sums over all four lane quarters (fixed order)
    u32x4_t xb[2 * GPW];
    float X[GPW];
    {
        const bool have = r < a.M;
        const uint16_t* xrow = a.x + (size_t)(have ? r : 0) * a.K + 64 * g0;
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            float s0 = 0.f, s1 = 0.f;
            xb[2 * g] = stage_x_operand<BITS>(xrow, 2 * g, c, s0);
            xb[2 * g + 1] = stage_x_operand<BITS>(xrow, 2 * g + 1, c, s1);
            if (!have) {
                xb[2 * g] = xb[2 * g + 1] = u32x4_t{0u, 0u, 0u, 0u};
                s0 = s1 = 0.f;
            }
            const float v = s0 + s1;
            const float v16 = __shfl_xor(v, 16);
            const float p = (c & 1) ? v16 + v : v + v16;
            const float p32 = __shfl_xor(p, 32);
            X[g] = (c & 2) ? p32 + p : p + p32;
        }
    }

    uint32_t cmask = AffineMma<BITS>::MASK, cbias = 0x43004300u;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+v"(cbias));
    const bool hi8 = (lane & 8) != 0;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KPW; ++p) {
        // pc[0][t]: codes of k-step t of the block, pc[1][t]: k-step 4 + t
        uint32_t pc[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l0 = wa[p][0][i], l1 = wa[p][1][i];
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l0, 0x128, 0xF, 0xF, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)l1, 0x128, 0xF, 0xF, false);
            pc[0][i] = hi8 ? r1 : l0;
            pc[1][i] = hi8 ? l1 : r0;
        }
        transpose4x4_rows(pc[0]);
        transpose4x4_rows(pc[1]);
#pragma unroll
        for (int gi = 0; gi < GPK; ++gi) {
            const int g = p * GPK + gi;          // group within the wavefront's range
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
            f32x4_t dg = mfma16x16x32(A0, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
            dg = mfma16x16x32(A1, xb[2 * g + 1], dg);
            if constexpr (BITS == 8) {
                f32x4_t dh = mfma16x16x32(H0, xb[2 * g], f32x4_t{0.f, 0.f, 0.f, 0.f});
                dh = mfma16x16x32(H1, xb[2 * g + 1], dh);
#pragma unroll
                for (int i = 0; i < 4; ++i) dg[i] = fmaf(16.0f, dh[i], dg[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sh = sw[i][g >> 1], bh = bw[i][g >> 1];
                const float s = __uint_as_float((g & 1) ? (sh & 0xFFFF0000u) : (sh << 16));
                const float bi = __uint_as_float((g & 1) ? (bh & 0xFFFF0000u) : (bh << 16));
                acc[i] = fmaf(s, dg[i], fmaf(fmaf(-OFF, s, bi), X[g], acc[i]));
            }
        }
    }

    // fixed-order sum of the k-splits: every wavefront stores its partial
    // tile (rows of 65 floats: conflict-free reads below), then every thread
    // adds one output's partials in order 0, 1, ..., nks-1 and stores it
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_red[(size_t)(wave * 4 + i) * 65 + lane] = acc[i];
    __syncthreads();
    // output (m, n0 + n16) lives in lane (n16 / 4) * 16 + m, element n16 % 4
    for (int o = threadIdx.x; o < 256; o += blockDim.x) {
        const int m = o >> 4, n16 = o & 15;
        const int j0 = (n16 & 3) * 65 + (n16 >> 2) * 16 + m;
        float v = lds_red[j0];
        for (int w = 1; w < nks; ++w) v += lds_red[(size_t)(w * 4) * 65 + j0];
        const int64_t n = n0 + n16;
        if (m >= a.M || n >= a.N) continue;
        const size_t oi = (size_t)m * a.N + n;
        if (a.out_f32) reinterpret_cast<float*>(a.y)[oi] = v;
        else reinterpret_cast<uint16_t*>(a.y)[oi] = f32_to_bf16_rne(v);
    }
}

// k-blocks per wavefront: the smallest of 1, 2, 4 that splits the row's
// 128-byte k-blocks over at most 16 wavefronts, with at most 8 groups per
// wavefront (their x^T operands take 8 registers each; 0 if none fits).
inline int affine_split_kpw(int bits, int K)
{
    if (!(bits == 2 || bits == 4 || bits == 8) || K % 64 != 0 || (K * bits) % 1024 != 0) return 0;
    const int kbl = K * bits / 1024;
    for (int kpw : {1, 2, 4})
        if (kbl % kpw == 0 && kbl / kpw <= kAffineSplitMaxWaves) return kpw * (16 / bits) <= 8 ? kpw : 0;
    return 0;
}

template <int BITS, int KPW>
hipError_t launch_affine_split_one(const ProjArgs& a, hipStream_t s)
{
    if (a.M > 32) return hipErrorInvalidValue;
    const int nks = (a.K * BITS / 1024) / KPW;
    const int64_t tiles = ((int64_t)a.N + 15) / 16;
    const size_t lds = (size_t)nks * 4 * 65 * 4;
    // M = 17..32 runs once per 16-column block, and with at most half as many
    // row tiles as CUs M = 9..16 once per 8-column block (the two blocks of a
    // tile on one XCD).
    if (a.M > 16) {
        const int64_t blocks = (tiles + 7) / 8 * 16;
        hipLaunchKernelGGL((affine_split_kernel<BITS, KPW, 16>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
        return hipGetLastError();
    }
    if (a.M > 8) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (2 * tiles <= cus) {
            const int64_t blocks = (tiles + 7) / 8 * 16;
            hipLaunchKernelGGL((affine_split_kernel<BITS, KPW, 8>), dim3((unsigned)blocks), dim3(64 * nks), lds, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((affine_split_kernel<BITS, KPW>), dim3((unsigned)tiles), dim3(64 * nks), lds, s, a);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_affine_split_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    (void)c;
    constexpr int GPK = AffineMma<BITS>::GPK;
    switch (affine_split_kpw(BITS, a.K)) {
        case 1: return launch_affine_split_one<BITS, 1>(a, s);
        case 2:
            if constexpr (2 * GPK <= 8) return launch_affine_split_one<BITS, 2>(a, s);
            else return hipErrorInvalidValue;
        case 4:
            if constexpr (4 * GPK <= 8) return launch_affine_split_one<BITS, 4>(a, s);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
