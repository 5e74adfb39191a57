// Matrix-core GEMM for affine codes of 2 to 8 bits at any M (prompt chunks:
// M > 32 rows of activations), on gfx950.
//
//   y[m, n] = sum_k x[m, k] (s[n, g] q[n, k] + b[n, g]),   g = k / 64
//
// in the factored form sum_g s[n,g] D[m,n,g] + sum_g (b[n,g] X[m,g] -
// s[n,g] D0[m,g]) with X the group sums of x, evaluated in fp32:
//
//   * D is the group's dot product of x with the codes as the matrix core
//     computes it (v_mfma_f32_16x16x32_bf16, two k-steps per group).  For 2
//     to 7 bits a code goes into a bf16 mantissa as 128 + q (mask placement,
//     no lookup, as in the decode kernels); 8-bit codes are converted to bf16
//     exactly (every integer up to 256 is a bf16), so D carries no offset.
//   * D0 is that offset, 128 X, as the matrix core computes it for all-zero
//     codes (the same two MFMAs on the same x operands), so a group of zero
//     codes gives D == D0 bit for bit.  No offset for 8 bits.
//   * Per group and output the wavefront adds s D into its fp32 tile: one FMA.
//   * The code-independent terms sum_g b X and - sum_g s D0 are a contraction
//     over the groups that the matrix core does once per tile, 32 groups per
//     MFMA: A = the rows' biases (bf16, exact) or negated scales, B = X or D0
//     split into three bf16 pieces (hi, mid, lo: X = hi + mid + lo exactly for
//     a normal fp32 X), products exact in fp32.
//
// A pre-pass over x (gemm_prep_kernel) writes, into the caller's workspace,
// the x^T B operands of every (16-row block, group, k-step) in the width's k
// order (1 KB each, laid out exactly as the main kernel keeps them in LDS)
// and the six pieces per (row, group).
//
// Main kernel (affine_gemm_kernel): a workgroup of 8 wavefronts owns a tile
// of 64 WN rows of W by 64 rows of x and walks K one group per stage; with
// WK > 1 the K range is split into WK chunks, one per slice of WN
// wavefronts.  Wavefront (wn, kc) owns rows 64 wn .. + 63 of the tile in
// chunk kc: a 64 x 64 output tile, 4 x 4 MFMA tiles of 16 x 16.
//   * Codes are private to the wavefront that owns their rows, so they go
//     from HBM straight into its registers: per 16-row block a lane reads
//     the words holding its window (lane quarter c: codes 16c .. 16c + 15
//     of the group).  The x operands are shared by the WN wavefronts of a
//     chunk: each stage's 1 KB blocks are loaded by all threads and written
//     to one of two LDS buffers.  A scale per lane (its row's) goes through
//     a wavefront-private LDS table to the lanes holding that row's outputs.
//   * Loads run D stages ahead of the arithmetic in a ring of register sets
//     indexed with constants only (the loop is unrolled D + 1 times); D is
//     as large as the registers allow beside the tile.  One barrier a stage.
//   * Per stage and 16-row block: the two A operands from the code window,
//     4 + 4 MFMAs into fresh 16 x 16 tiles, 16 FMAs of the scale into the
//     running sums.  All loads are plain buffer loads the compiler sees, so
//     its own waits cover them.  (Copies straight into LDS were measured
//     slower here: their issue rate, not HBM, bounded the stage.)
// The chunk partials of a tile are summed through LDS in chunk order
// (fixed: no result depends on the other rows of x), then stored as fp32 or
// RNE bf16.  Consecutive tiles (same rows of W, successive blocks of x) go to
// one XCD, so a tile's codes are read from HBM once and then hit in its L2.
//
// Format: TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2
// to 8 bits in groups of 64" (MLX affine mode, groups of 64); the same page
// notes that its 8-bit modules have no prompt GEMM and run prompt chunks on
// the decode tiles, 16 rows at a time.
#pragma once

#include "affine_tile.h"
#include "host_query.h"
#include "kernels.h"

namespace aqg {

namespace detail {

constexpr int kGemmWaves = 8;   // wavefronts per workgroup

// ------------------------------------------------------------ k orders

// Element e (0..15) of a lane's 16-value x window held as 8 bf16 pairs.
template <int E>
__device__ __forceinline__ uint32_t win_elem(const uint32_t (&v)[8])
{
    return (E & 1) ? (v[E >> 1] >> 16) : (v[E >> 1] & 0xFFFFu);
}

// x^T operand of k-step H from a lane's window (x at 16c .. 16c + 15 of the
// group), in the k order of the width's A operands:
//   2 bits: 4H + {0, 8, 1, 9, 2, 10, 3, 11}   (codes2_to_bf16)
//   4 bits: 8H + {0, 4, 1, 5, 2, 6, 3, 7}     (codes4_to_bf16)
//   other widths: 8H + {0 .. 7}, natural
template <int BITS, int H>
__device__ __forceinline__ u32x4_t gemm_x_operand(const uint32_t (&v)[8])
{
    u32x4_t o;
    static_for<0, 4>([&](auto Tc) __attribute__((always_inline)) {
        constexpr int t = decltype(Tc)::value;
        if constexpr (BITS == 2) {
            o[t] = win_elem<4 * H + t>(v) | (win_elem<4 * H + t + 8>(v) << 16);
        } else if constexpr (BITS == 4) {
            o[t] = win_elem<8 * H + t>(v) | (win_elem<8 * H + t + 4>(v) << 16);
        } else {
            o[t] = v[4 * H + t];
        }
    });
    return o;
}

// Eight 8-bit codes (dwords a, b; byte i = code i) as exact bf16 pairs in
// natural order (q0, q1), (q2, q3), (b0, b1), (b2, b3).
__device__ __forceinline__ u32x4_t codes8_exact_bf16(uint32_t a, uint32_t b)
{
    auto pair = [](uint32_t w, int sh) __attribute__((always_inline)) {
        const float lo = (float)((w >> sh) & 0xFFu);
        const float hi = (float)((w >> (sh + 8)) & 0xFFu);
        return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    };
    return u32x4_t{pair(a, 0), pair(a, 16), pair(b, 0), pair(b, 16)};
}

// ------------------------------------------------------------ pre-pass

// Truncation of an fp32 to its top 8 significant bits (a bf16 value).
__device__ __forceinline__ float bf16_trunc(float f) { return __uint_as_float(__float_as_uint(f) & 0xFFFF0000u); }

// One wavefront per (16-row block mt of x, group g < Gp): lane (c, r) takes
// row 16 mt + r and x[64 g + 16 c .. + 15].  Writes the two x operands of
// the group (g < G), and with c == 0 the six (three) pieces of (row, g);
// rows past M and groups past G give zeros.
template <int BITS>
__global__ void __launch_bounds__(256) gemm_prep_kernel(GemmArgs a)
{
    const int lane = threadIdx.x & 63;
    const int c = lane >> 4, r = lane & 15;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t units = (int64_t)(a.Mp / 16) * a.Gp;
    if (w >= units) return;   // wave-uniform
    const int mt = (int)(w / a.Gp), g = (int)(w % a.Gp);
    const int m = 16 * mt + r;
    const bool have = m < a.M && g < a.G;

    uint32_t v[8];
    if (have) {
        const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)m * a.K + 64 * g + 16 * c);
        const uint4 p = src[0], q = src[1];
        v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
        v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0u;
    }
    const u32x4_t b0 = gemm_x_operand<BITS, 0>(v);
    const u32x4_t b1 = gemm_x_operand<BITS, 1>(v);
    if (g < a.G) {
        uint4* dst = reinterpret_cast<uint4*>(a.xp) + (((int64_t)mt * a.G + g) * 2) * 64 + lane;
        dst[0] = make_uint4(b0[0], b0[1], b0[2], b0[3]);
        dst[64] = make_uint4(b1[0], b1[1], b1[2], b1[3]);
    }

    // X: the window summed in a fixed order, then over the lane quarters
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = bf16_to_f32(v[i] & 0xFFFFu) + bf16_to_f32(v[i] >> 16);
    float part = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
    const float p16 = __shfl_xor(part, 16);
    const float h = (c & 1) ? p16 + part : part + p16;
    const float h32 = __shfl_xor(h, 32);
    const float X = (c & 2) ? h32 + h : h + h32;

    float vals[6];
    vals[0] = bf16_trunc(X);
    const float rx = X - vals[0];
    vals[1] = bf16_trunc(rx);
    vals[2] = rx - vals[1];
    if constexpr (BITS != 8) {
        const u32x4_t Z = u32x4_t{kZeroCodePair, kZeroCodePair, kZeroCodePair, kZeroCodePair};
        f32x4_t d = mfma16x16x32(Z, b0, f32x4_t{0.f, 0.f, 0.f, 0.f});
        d = mfma16x16x32(Z, b1, d);
        const float D0 = d[0];   // every row of the all-128 A operand is the same
        vals[3] = bf16_trunc(D0);
        const float rd = D0 - vals[3];
        vals[4] = bf16_trunc(rd);
        vals[5] = rd - vals[4];
    }
    if (c == 0) {
#pragma unroll
        for (int p = 0; p < gemm_pieces(BITS); ++p)
            a.pieces[((int64_t)p * a.Mp + m) * a.Gp + g] = f32_to_bf16_rne(vals[p]);
    }
}

// ------------------------------------------------------------ main kernel

template <int BITS, int WN, int WK>
struct GemmLayout {
    static constexpr int NW = WN * WK;                    // wavefronts
    static constexpr int NT = 64 * NW;                    // threads
    static constexpr int MB = kGemmTileM / 16;            // 16-column blocks of a tile
    static constexpr int ROWS = 64 * WN;                  // rows of W per tile
    static constexpr int GB = 8 * BITS;                   // code bytes per row and group
    static constexpr int NWW = (2 * BITS + 3) / 4;        // code words a lane reads per row and group
    static constexpr int XOP = WK * MB * 2 * 1024;        // x operand bytes per stage
    static constexpr int XLD = XOP / 16 / NT;             // 16-byte x loads per thread per stage
    static constexpr int TAB = NW * 2 * 8 * 64 * 4;       // per-wavefront fp32 scale tables [2][8][64]
    static constexpr int RED = (WK - 1) * WN * 64 * 64 * 4;   // chunk partials (over the x buffers)
    static constexpr int RING = 2 * XOP > RED ? 2 * XOP : RED;
    static constexpr size_t LDS = (size_t)RING + TAB;
    static_assert(NW == kGemmWaves, "eight wavefronts per workgroup");
    static_assert(XOP % (16 * NT) == 0, "x loads split evenly over the threads");
    static_assert(LDS <= 160 * 1024, "LDS of one CU");
};

// The lane's code window (codes 16c .. 16c + 15 of a group) from the words
// it read: NWW consecutive words of the row starting at word (16 b c) / 32
// of the group, the window starting at bit sh = (16 b c) % 32 (0, or 16
// for odd widths and odd c).  The A operands of the group's two k-steps.
// m = field mask, mh = m << 16, cb = 0x43004300, opaque registers.
template <int BITS>
__device__ __forceinline__ void gemm_a_from_words(const uint32_t (&w)[GemmLayout<BITS, 8, 1>::NWW], uint32_t sh,
                                                  uint32_t m, uint32_t mh, uint32_t cb, u32x4_t& a0, u32x4_t& a1)
{
    if constexpr (BITS == 2) {
        a0 = codes2_to_bf16(w[0], 0, m, cb);
        a1 = codes2_to_bf16(w[0], 1, m, cb);
    } else if constexpr (BITS == 4) {
        a0 = codes4_to_bf16(w[0], m, cb);
        a1 = codes4_to_bf16(w[1], m, cb);
    } else if constexpr (BITS == 8) {
        a0 = codes8_exact_bf16(w[0], w[1]);
        a1 = codes8_exact_bf16(w[2], w[3]);
    } else {
        constexpr int NWN = AffineTileWidth<BITS>::NWN;
        static_assert(NWN <= GemmLayout<BITS, 8, 1>::NWW, "the window fits the words read");
        uint32_t wn[NWN];
#pragma unroll
        for (int i = 0; i + 1 < NWN; ++i) wn[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
        wn[NWN - 1] = w[NWN - 1] >> sh;   // only its low 16 bits belong to the window when sh = 16
        a0 = codes_window_to_bf16<BITS, 0>(wn, m, mh, cb);
        a1 = codes_window_to_bf16<BITS, 1>(wn, m, mh, cb);
    }
}

// Eight consecutive bf16 of a row of an [N][G] array, groups g0 .. g0 + 7,
// zero past the row's end (G) or for a row past N.  even: G is even (dword
// loads are aligned).
__device__ __forceinline__ u32x4_t load8_groups(const uint16_t* arr, int64_t n, int N, int G, int g0, bool even)
{
    u32x4_t o = u32x4_t{0u, 0u, 0u, 0u};
    if (n >= N || g0 >= G) return o;
    const uint16_t* p = arr + n * G + g0;
    if (even && g0 + 8 <= G) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        o = u32x4_t{q[0], q[1], q[2], q[3]};
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = g0 + i < G ? (uint32_t)p[i] : 0u;
            o[i >> 1] |= (i & 1) ? (v << 16) : v;
        }
    }
    return o;
}

// One stage's loads of a thread: the code words of its 4 rows (one per
// 16-row block), its x operand pieces and its row's scale.
template <int BITS, int WK>
struct GemmStage {
    uint32_t cw[4][GemmLayout<BITS, 8, 1>::NWW];
    u32x4_t xo[WK];
    uint32_t sc;
};

template <int BITS, int WN, int WK, int D>
__global__ void __launch_bounds__(64 * kGemmWaves) affine_gemm_kernel(GemmArgs a)
{
    using L = GemmLayout<BITS, WN, WK>;
    constexpr int MB = L::MB;
    constexpr int NWW = L::NWW;
    constexpr int NP = gemm_pieces(BITS);
    constexpr int R = D + 1;   // stage register sets: the one in use and D in flight
    extern __shared__ __attribute__((aligned(16))) char gemm_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4, r = lane & 15;
    const int wn = wave % WN, kc = wave / WN;

    // tile of this workgroup: consecutive tiles (same rows of W, successive
    // 64-row blocks of x) go to the workgroups of one XCD
    const int TM = a.Mp / kGemmTileM;
    const int64_t T = (((int64_t)a.N + L::ROWS - 1) / L::ROWS) * TM;
    const int64_t bid = blockIdx.x;
    const int64_t tile = (gridDim.x % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
    const int64_t n0 = (tile / TM) * L::ROWS;
    const int m0 = (int)(tile % TM) * kGemmTileM;
    // blockIdx.y: this workgroup's share of the groups when the tile is split
    // over a.ks workgroups (their partial products are summed afterwards)
    const int GC = a.G / (WK * a.ks);   // groups (stages) per chunk
    const int zb = (int)blockIdx.y * WK * GC;   // first group of this workgroup
    const int g0 = zb + kc * GC;        // this wavefront's first group
    const int64_t row_bytes = (int64_t)a.K * BITS / 8;
    const int64_t rows_here = (int64_t)a.N - n0 < L::ROWS ? (int64_t)a.N - n0 : L::ROWS;

    // rows past N and x blocks past the workspace read as zeros
    const __amdgpu_buffer_rsrc_t rw =
        tile_rsrc(reinterpret_cast<const char*>(a.wq) + n0 * row_bytes, rows_here * row_bytes);
    const int64_t xp0 = (int64_t)(m0 / 16) * a.G * 2048;   // bytes
    const __amdgpu_buffer_rsrc_t rx = tile_rsrc(reinterpret_cast<const char*>(a.xp) + xp0, (int64_t)MB * a.G * 2048);
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.scales + n0 * a.G, rows_here * a.G * 2);

    // code words: row 64 wn + 16 t + r of the tile, word (16 b c) / 32 of
    // the group; x pieces: thread j loads piece j of each chunk's
    // [mb][k-step][lane] block; scale: row 64 wn + lane.  The lane's part
    // (row, position in the group) is the vector offset, which the range
    // check covers (rows past N read zeros).  For 2-, 4- and 8-bit codes the
    // group's offset (and the stage's offsets of x and the scales), the same
    // for the whole wavefront, is the scalar offset, so a stage costs no
    // address arithmetic; for the other widths (groups of 24 to 56 bytes)
    // that measured much slower (5 bits, 14336 x 4096 at 512 rows: 231 us
    // against 138 us), so there it stays in the vector offset.
    constexpr bool SOFF = BITS == 2 || BITS == 4 || BITS == 8;
    const int bit0 = 16 * BITS * c;
    const uint32_t sh = (uint32_t)(bit0 & 31);
    const uint32_t code_off = (uint32_t)((64 * wn + r) * row_bytes + (SOFF ? 0 : (int64_t)g0 * L::GB) + 4 * (bit0 >> 5));
    const uint32_t code_tstride = (uint32_t)(16 * row_bytes);
    const int j = threadIdx.x;
    const int jmb = j / 128, jh = (j / 64) % 2, jl = j % 64;
    const uint32_t x_off = (uint32_t)(((jmb * a.G + zb) * 2 + jh) * 1024 + jl * 16);
    // scales: 8-group windows, one 8-row block a stage (see load)
    const uint32_t s_off = (uint32_t)((((int64_t)64 * wn + (lane >> 3)) * a.G + (lane & 7)) * 2);
    const uint32_t s_rb = (uint32_t)(8 * a.G * 2);   // bytes per 8 rows

    auto load = [&](int i, GemmStage<BITS, WK>& st) __attribute__((always_inline)) {
        const uint32_t cs = SOFF ? (uint32_t)((g0 + i) * L::GB) : 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t vo = code_off + (SOFF ? 0u : (uint32_t)(i * L::GB)) + t * code_tstride;
            if constexpr (BITS == 4) {          // 8 bytes at 8 c: one aligned 8-byte load
                const u32x2v_t v = __builtin_bit_cast(u32x2v_t, __builtin_amdgcn_raw_buffer_load_b64(rw, vo, cs, 0));
                st.cw[t][0] = v[0];
                st.cw[t][1] = v[1];
            } else if constexpr (BITS == 8) {   // 16 bytes at 16 c
                const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, vo, cs, 0));
#pragma unroll
                for (int q = 0; q < 4; ++q) st.cw[t][q] = v[q];
            } else {
#pragma unroll
                for (int q = 0; q < NWW; ++q)
                    st.cw[t][q] = __builtin_amdgcn_raw_buffer_load_b32(rw, vo + 4 * q, cs, 0);
            }
        }
#pragma unroll
        for (int q = 0; q < WK; ++q)
            st.xo[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                rx, x_off + (SOFF ? 0u : (uint32_t)((q * GC + i) * 2048)), SOFF ? (uint32_t)((q * GC + i) * 2048) : 0u, 0));
        // the scales of the next 8-group window, 8 rows a stage: lane l takes
        // row 8 (i % 8) + l / 8 of the wavefront's rows and group l % 8 of
        // window i / 8 + 1, so one load covers 8 rows of 16 bytes (not 64
        // rows); the row stays in the vector offset (range-checked)
        const uint32_t sg = (uint32_t)(2 * (g0 + 8 * (i / 8 + 1)));
        st.sc = __builtin_amdgcn_raw_buffer_load_b16(rs, s_off + (uint32_t)(i % 8) * s_rb + (SOFF ? 0u : sg),
                                                     SOFF ? sg : 0u, 0);
    };
    // window 0 before the first stage
    auto load_window0 = [&](uint32_t (&w0)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
            w0[b] = __builtin_amdgcn_raw_buffer_load_b16(rs, s_off + (uint32_t)b * s_rb + (SOFF ? 0u : (uint32_t)(2 * g0)),
                                                         SOFF ? (uint32_t)(2 * g0) : 0u, 0);
    };
    auto put_x = [&](int buf, const GemmStage<BITS, WK>& st) __attribute__((always_inline)) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(gemm_lds + buf * L::XOP);
#pragma unroll
        for (int q = 0; q < WK; ++q) dst[q * L::NT + j] = st.xo[q];
    };

    f32x4_t acc[4][MB];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint32_t cmask = BITS == 2 ? 0x00030003u : BITS == 4 ? 0x000F000Fu : AffineTileWidth<BITS>::MASK;
    uint32_t cmaskh = AffineTileWidth<BITS>::MASK << 16, cbias = kZeroCodePair;
    asm volatile("" : "+s"(cmask));      // no instruction: only hides the constants
    asm volatile("" : "+s"(cmaskh));
    asm volatile("" : "+v"(cbias));

    // the wavefront's scales [window parity][group of the window][row]
    float* tab = reinterpret_cast<float*>(gemm_lds + L::RING) + wave * (2 * 8 * 64);

    // group i: both k-steps of each 16 x 16 tile, then the group's scale
    // into the running sums, one 16-row block at a time
    auto compute = [&](int i, const GemmStage<BITS, WK>& st) __attribute__((always_inline)) {
        // this stage's block of the next window, then the scales of group i
        // (written 8 or more stages ago, by this wavefront: LDS operations of
        // one wavefront take effect in program order)
        tab[((i / 8 + 1) & 1) * 512 + (lane & 7) * 64 + 8 * (i % 8) + (lane >> 3)] = __uint_as_float(st.sc << 16);
        const float* tg = tab + ((i / 8) & 1) * 512 + (i % 8) * 64;
        f32x4_t S[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) S[t][v] = tg[16 * t + 4 * c + v];
        const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(gemm_lds + (i & 1) * L::XOP) + kc * 512;
        u32x4_t xb[MB][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) xb[mb][hh] = xs[(mb * 2 + hh) * 64 + lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4_t a0, a1;
            gemm_a_from_words<BITS>(st.cw[t], sh, cmask, cmaskh, cbias, a0, a1);
            f32x4_t d[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) d[mb] = mfma16x16x32(a0, xb[mb][0], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) d[mb] = mfma16x16x32(a1, xb[mb][1], d[mb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][mb][v] = fmaf(S[t][v], d[mb][v], acc[t][mb][v]);
        }
    };

    // D stages in flight: the loads of group i + D go out before group i is
    // computed; group i + 1's x pieces go to LDS after it.  The ring is
    // indexed with constants only (unrolled R times), so it stays in
    // registers.  Every load is unconditional (a stage past the chunk's
    // last group reloads that group, a cache hit): a load under a branch
    // makes the compiler wait for every load in flight where the paths
    // join, which would drain the ring at each stage.  Only the arithmetic
    // of the stages past the end is skipped, and the LDS writes after it
    // go to the buffer nobody reads any more.
    // (issued stage by stage, in the loop's order: the wait for a stage's
    // data counts the loads issued after it, and where the first pass joins
    // the loop the compiler takes the smaller count of the two paths)
    uint32_t w0[8];
    load_window0(w0);
    __builtin_amdgcn_sched_barrier(0);
    GemmStage<BITS, WK> ring[R];
    static_for<0, D>([&](auto Uc) __attribute__((always_inline)) {
        constexpr int u = decltype(Uc)::value;
        load(u < GC ? u : GC - 1, ring[u]);
        __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int b = 0; b < 8; ++b) tab[(lane & 7) * 64 + 8 * b + (lane >> 3)] = __uint_as_float(w0[b] << 16);
    put_x(0, ring[0]);
    __syncthreads();
    for (int base = 0; base < GC; base += R) {
        static_for<0, R>([&](auto Uc) __attribute__((always_inline)) {
            constexpr int u = decltype(Uc)::value;
            const int i = base + u;
            load(i + D < GC ? i + D : GC - 1, ring[(u + D) % R]);
            if (i < GC) compute(i, ring[u]);   // uniform over the workgroup
            put_x((i + 1) & 1, ring[(u + 1) % R]);
            __syncthreads();
        });
    }

    // sum_g (b X - s D0): units (32-group block j, piece p), chunk kc taking
    // p = kc, kc + WK, ...; all groups, in the first share of a split tile
    if (blockIdx.y == 0) {
        const bool even = (a.G & 1) == 0;
        const int NJ = a.Gp / 32;
        for (int j = 0; j < NJ; ++j) {
            const int g0 = 32 * j + 8 * c;
            u32x4_t ab[4], as[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t n = n0 + 64 * wn + 16 * t + r;
                ab[t] = load8_groups(a.biases, n, a.N, a.G, g0, even);
                as[t] = load8_groups(a.scales, n, a.N, a.G, g0, even);
                as[t] ^= u32x4_t{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            }
            for (int p = kc; p < NP; p += WK) {
                u32x4_t bp[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    bp[mb] = *reinterpret_cast<const u32x4_t*>(
                        a.pieces + ((int64_t)p * a.Mp + m0 + 16 * mb + r) * a.Gp + g0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[t][mb] = mfma16x16x32(p < 3 ? ab[t] : as[t], bp[mb], acc[t][mb]);
            }
        }
    }

    // chunk partials, summed in chunk order
    if constexpr (WK > 1) {
        // every wavefront is done with the x buffers (the loop ends with a barrier)
        f32x4_t* red = reinterpret_cast<f32x4_t*>(gemm_lds);
        if (kc > 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    red[(((kc - 1) * WN + wn) * 16 + t * MB + mb) * 64 + lane] = acc[t][mb];
        }
        __syncthreads();
        if (kc > 0) return;
#pragma unroll
        for (int k2 = 1; k2 < WK; ++k2)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[t][mb] += red[(((k2 - 1) * WN + wn) * 16 + t * MB + mb) * 64 + lane];
    }

    // store: lane (c, r) holds rows n .. n + 3 of column m of each 16 x 16 tile
    // (a split tile: this share's fp32 partial products)
    const bool vec = (a.N & 3) == 0;
    if (a.ks > 1) {
        float* part = a.part + (size_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t n = n0 + 64 * wn + 16 * t + 4 * c;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = m0 + 16 * mb + r;
                if (m >= a.M || n >= a.N) continue;
                float* y = part + (int64_t)m * a.N + n;
                const f32x4_t v = acc[t][mb];
                if (vec) {
                    *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) y[e] = v[e];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t n = n0 + 64 * wn + 16 * t + 4 * c;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = m0 + 16 * mb + r;
            if (m >= a.M || n >= a.N) continue;
            const int64_t o = (int64_t)m * a.N + n;
            const f32x4_t v = acc[t][mb];
            if (a.out_f32) {
                float* y = static_cast<float*>(a.y) + o;
                if (vec) {
                    *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) y[e] = v[e];
                }
            } else {
                uint16_t* y = static_cast<uint16_t*>(a.y) + o;
                const uint16_t h0 = f32_to_bf16_rne(v[0]), h1 = f32_to_bf16_rne(v[1]);
                const uint16_t h2 = f32_to_bf16_rne(v[2]), h3 = f32_to_bf16_rne(v[3]);
                if (vec) {
                    *reinterpret_cast<uint2*>(y) = make_uint2(h0 | ((uint32_t)h1 << 16), h2 | ((uint32_t)h3 << 16));
                } else {
                    const uint16_t h[4] = {h0, h1, h2, h3};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < a.N) y[e] = h[e];
                }
            }
        }
    }
}

// ------------------------------------------------------------ host side

// Sum of the ks partial products of every output, in share order 0, 1, ...,
// ks - 1, then the output rounding.
// (a template, like every kernel of this header, so each width's unit
// instantiates its own copy)
template <int BITS>
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmArgs a)
{
    const int64_t MN = (int64_t)a.M * a.N;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float v = a.part[i];
    for (int z = 1; z < a.ks; ++z) v += a.part[(int64_t)z * MN + i];
    if (a.out_f32) static_cast<float*>(a.y)[i] = v;
    else static_cast<uint16_t*>(a.y)[i] = f32_to_bf16_rne(v);
}

// Stages in flight: as many as the registers allow beside the 64 x 64 tile
// (a stage is 4 NWW code words, WK x pieces and a scale per lane).
template <int BITS, int WK>
constexpr int gemm_depth()
{
    constexpr int regs = 4 * GemmLayout<BITS, 8, 1>::NWW + 4 * WK + 1;
    constexpr int d = 60 / regs;
    return WK >= 4 ? 1 : d > 4 ? 4 : d;
}

template <int BITS, int WN, int WK>
hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t s)
{
    using L = GemmLayout<BITS, WN, WK>;
    auto fn = affine_gemm_kernel<BITS, WN, WK, gemm_depth<BITS, WK>()>;
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(fn), L::LDS);
    if (e != hipSuccess) return e;
    const int64_t T = (((int64_t)a.N + L::ROWS - 1) / L::ROWS) * (a.Mp / kGemmTileM);
    if (T > 0x7FFFFFFF || a.ks < 1 || a.G % (WK * a.ks) != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)T, (unsigned)a.ks), dim3(64 * kGemmWaves), L::LDS, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.ks == 1) return e;
    const int64_t MN = (int64_t)a.M * a.N;
    hipLaunchKernelGGL(gemm_reduce_kernel<BITS>, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_affine_gemm_impl(const GemmArgs& a, hipStream_t s)
{
    const int64_t units = (int64_t)(a.Mp / 16) * a.Gp;
    hipLaunchKernelGGL(gemm_prep_kernel<BITS>, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const GemmCfg g{a.wn, 8 / a.wn};
    if (g.wn == 8) return launch_gemm_cfg<BITS, 8, 1>(a, s);
    if (g.wn == 4) return launch_gemm_cfg<BITS, 4, 2>(a, s);
    return launch_gemm_cfg<BITS, 2, 4>(a, s);
}

}  // namespace detail
}  // namespace aqg
