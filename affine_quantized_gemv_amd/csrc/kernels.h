// Host-side interface between the C ABI (abi.hip) and the kernels
// (kernels.hip, proj_b*.hip, mfma_*.hip).  Not installed; not part of the
// public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aqg {

constexpr int kMaxSegments = 4;   // projections of one multi-projection launch

// Arguments of one projection launch.  Pointers are device pointers.
struct ProjArgs {
    const uint16_t* x;       // bf16 [M][K]
    const void* w0;          // dense W, affine Wq words, or SwiGLU Wg
    const void* w1;          // SwiGLU Wu (else null)
    const uint16_t* scales;  // affine: bf16 [N][K/64] (SwiGLU: of Wg)
    const uint16_t* biases;  // affine: bf16 [N][K/64] (SwiGLU: of Wg)
    const uint16_t* scales1; // affine SwiGLU: scales of Wu (else null)
    const uint16_t* biases1; // affine SwiGLU: biases of Wu (else null)
    void* y;                 // bf16 or f32 [M][N]
    int M, N, K;
    int KT;                  // K elements staged in LDS per tile
    int lpr_log2;            // VALU/stream paths: log2 of lanes that share one weight row
    int ksplit_log2;         // MFMA path: log2 of wavefronts splitting K per row group
    int out_f32;             // 1: store fp32, 0: store bf16 (RNE)
    int64_t tpw;             // stream path: row tiles per super-tile
    int64_t tmax;            // stream path: most row tiles any wavefront finishes
    // Row argmax instead of a store (null: store y).  The kernel writes one
    // (value, index) partial per output row m for each of its producers
    // (wavefronts or workgroups, per kernel) to amx[m * amx_slots + producer];
    // a producer with no rows writes (-inf, INT_MAX).  amx_slots: producers
    // the buffer holds per row (a launch that needs more fails with
    // hipErrorInvalidValue); the launcher reports the producers it launched
    // through the host pointer amx_producers.
    void* amx;
    int64_t amx_slots;
    int64_t* amx_producers;
    // Several projections of one x in one launch (nseg > 1): the kernel sees
    // a virtual matrix whose rows are segment 0's rows, then segment 1's, ...
    // (N = the total); segment s starts at virtual row seg_row0[s] (a
    // multiple of 16, so no row tile straddles two segments), has its own
    // weights, scales and biases (affine) and its own output y_s [M][rows_s].
    // launch_proj fills a one-segment table (w0, scales, biases, y, N) when
    // nseg is 0, so the kernels read the table without a branch.
    int nseg;
    int64_t seg_row0[kMaxSegments + 1];
    const void* seg_w[kMaxSegments];
    const uint16_t* seg_scales[kMaxSegments];
    const uint16_t* seg_biases[kMaxSegments];
    void* seg_y[kMaxSegments];
};

// The segment table is read with constant indices only: a variable index
// into the kernel-argument arrays would make the compiler copy the whole
// argument block to private memory.

// Segment of virtual row n of a multi-projection launch (0 without).
__host__ __device__ inline int seg_of(const ProjArgs& a, int64_t n)
{
    int s = 0;
#pragma unroll
    for (int i = 1; i < kMaxSegments; ++i) s = ((i < a.nseg) & (n >= a.seg_row0[i])) ? i : s;
    return s;
}

// One field of segment s (a constant-index select).
template <class T>
__host__ __device__ inline T seg_pick(const T (&v)[kMaxSegments], int s)
{
    T r = v[0];
#pragma unroll
    for (int i = 1; i < kMaxSegments; ++i) r = s == i ? v[i] : r;
    return r;
}

// First row and row count of segment s.
__host__ __device__ inline int64_t seg_start(const ProjArgs& a, int s)
{
    int64_t r = a.seg_row0[0];
#pragma unroll
    for (int i = 1; i < kMaxSegments; ++i) r = s == i ? a.seg_row0[i] : r;
    return r;
}
__host__ __device__ inline int64_t seg_rows(const ProjArgs& a, int s)
{
    int64_t r = a.seg_row0[1] - a.seg_row0[0];
#pragma unroll
    for (int i = 1; i < kMaxSegments; ++i) r = s == i ? a.seg_row0[i + 1] - a.seg_row0[i] : r;
    return r;
}

// The matrix, scales, biases, output and row count of the projection holding
// virtual row n0 (a's own without segments), and n0 within that projection.
struct SegView {
    const void* w;
    const uint16_t* sc;
    const uint16_t* bi;
    void* y;
    int N;
    int64_t n0;
};
__host__ __device__ inline SegView seg_view(const ProjArgs& a, int64_t n0)
{
    const int s = seg_of(a, n0);
    return SegView{seg_pick(a.seg_w, s), seg_pick(a.seg_scales, s), seg_pick(a.seg_biases, s),
                   seg_pick(a.seg_y, s), (int)seg_rows(a, s), n0 - seg_start(a, s)};
}

enum Path { PATH_VALU = 0, PATH_MFMA = 1, PATH_STREAM = 2, PATH_PIECE = 3, PATH_MFMA_STREAM = 4, PATH_MFMA_SPLIT = 5, PATH_AFFINE_MFMA = 6,
            PATH_MFMA_TILE = 7, PATH_AFFINE_TILE = 8, PATH_AFFINE_SPLIT = 9, PATH_AFFINE_GEMM = 10, PATH_AFFINE_BURST = 11 };

// Launch geometry chosen for a call.
struct LaunchCfg {
    int path;       // PATH_*
    int MT;         // padded M (1, 2, 4, 8, 16, 32)
    int R;          // VALU: rows per lane; MFMA: 16-row tiles per row group (1 or 2)
    int lpr_log2;   // VALU: lanes per weight row = 2^lpr_log2 (<= 64)
    int ksplit_log2;  // MFMA: wavefronts splitting K per row group = 2^ksplit_log2
    int KT;         // K-tile in elements
    int xreg;       // stream/piece: x operands held in registers
    int pieces_per_lane;  // piece: 16-byte pieces per lane per row (1, 2, 3, 4, 8)
    int64_t tpw;    // stream: row tiles per wavefront
    int nwaves;     // waves per workgroup
    int blocks;     // workgroups
    size_t lds;     // dynamic LDS bytes
};

// Per-width VALU launchers, each instantiated in its own translation unit
// (proj_b*.hip) so the kernels compile in parallel.
template <int BITS, bool SWIGLU>
hipError_t launch_bits(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Per-width persistent streaming launchers (also in proj_b*.hip).
template <int BITS, bool SWIGLU>
hipError_t launch_stream(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Per-width persistent 16-byte-piece streaming launchers (piece_b*.hip):
// dense, SwiGLU and affine b = 2, 4, 8.
template <int BITS, bool SWIGLU>
hipError_t launch_piece(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Dense / SwiGLU matrix-core launcher (mfma_dense.hip).
template <bool SWIGLU>
hipError_t launch_mfma(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Persistent dense / SwiGLU matrix-core launcher for large N (mfma_stream.hip).
template <bool SWIGLU>
hipError_t launch_mfma_stream(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Dense / SwiGLU matrix-core launcher for small N, k split over one
// workgroup per 16-row tile (mfma_stream.hip).
template <bool SWIGLU>
hipError_t launch_mfma_split(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Dense matrix-core launcher for large N with whole tiles copied into LDS
// (mfma_tile.hip).
hipError_t launch_mfma_tile(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Affine matrix-core launcher with whole tiles copied into LDS, BITS = 2, 4
// or 8 (affine_tile_b*.hip).
template <int BITS>
hipError_t launch_affine_tile(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Affine matrix-core launcher for small N, k split over one workgroup per
// 16-row tile, BITS = 2..8 (affine_split.hip, affine_split_odd.hip; the
// fused SwiGLU over affine gate and up matrices in affine_split_swiglu.hip,
// affine_split_odd_swiglu.hip).
template <int BITS, bool SWIGLU>
hipError_t launch_affine_split(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Multi-tile affine matrix-core launcher at K = 4096 (1-4 row tiles per
// workgroup, all loads in flight at once; M = 17..32 as two 16-column
// launches), BITS = 2..8 (affine_burst.hip, affine_burst_odd.hip).
template <int BITS>
hipError_t launch_affine_burst(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Affine matrix-core launcher, BITS = 2, 4 or 8 (affine_mfma*.hip).
template <int BITS>
hipError_t launch_affine_mfma(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Row-argmax partials: the reduction over producers (argmax.hip).  part:
// int2 [M][slots] (value bits, index), producers 0 .. P-1 of each row.
hipError_t launch_argmax_final(const void* part, int64_t slots, int64_t P, int M, float* val, int* idx,
                               hipStream_t s);
// Row-argmax partials of y fp32 [M][N] in chunks of `chunk` columns:
// producers 0 .. ceil(N / chunk) - 1 of part [M][slots].
hipError_t launch_argmax_rows(const float* y, int M, int N, int chunk, void* part, int64_t slots, hipStream_t s);
// Whether the kernel of cfg writes row-argmax partials itself (else the
// caller runs the GEMV into fp32 and reduces the rows).
bool argmax_fused(const LaunchCfg& cfg);

// Arguments of one prompt GEMM (device pointers).  xp and pieces live in the
// caller's workspace and are written by the pre-pass.
struct GemmArgs {
    const uint16_t* x;        // bf16 [M][K]
    const uint32_t* wq;       // codes [N][K b / 32]
    const uint16_t* scales;   // bf16 [N][G]
    const uint16_t* biases;   // bf16 [N][G]
    void* y;                  // bf16 or f32 [M][N]
    uint16_t* xp;             // x operands [Mp / 16][G][2][64 lanes][8] bf16
    uint16_t* pieces;         // [NP][Mp][Gp] bf16: X hi, mid, lo, then D0 hi, mid, lo
    int M, N, K;
    int G;                    // groups per row, K / 64
    int Gp;                   // G rounded up to 32
    int Mp;                   // M rounded up to 64
    int out_f32;
    int wn;                   // 64-row blocks of W per tile: 8, 4 or 2 (8 / wn chunks of K)
    int ks;                   // groups split over ks workgroups per tile (1: no split)
    float* part;              // ks > 1: fp32 partial products [ks][M][N]
};

constexpr int kGemmTileM = 64;      // rows of x per tile

// Pieces per (row, group): X (3) and, with a code offset, D0 (3).
__host__ __device__ constexpr int gemm_pieces(int bits) { return bits == 8 ? 3 : 6; }

// Workspace of a prompt GEMM: the x operands (Mp K bf16), then, from the
// next 256-byte boundary, the pieces.
inline size_t gemm_workspace_base(int bits, int M, int K)
{
    const size_t Mp = ((size_t)M + kGemmTileM - 1) / kGemmTileM * kGemmTileM;
    const size_t G = (size_t)K / 64, Gp = (G + 31) / 32 * 32;
    const size_t xp = (Mp * K * 2 + 255) / 256 * 256;
    return xp + ((size_t)gemm_pieces(bits) * Mp * Gp * 2 + 255) / 256 * 256;
}
inline size_t gemm_pieces_offset(int M, int K)
{
    const size_t Mp = ((size_t)M + kGemmTileM - 1) / kGemmTileM * kGemmTileM;
    return (Mp * K * 2 + 255) / 256 * 256;
}

// Split of the 8 wavefronts of a prompt-GEMM workgroup: 64 WN rows of W per
// tile, K in WK chunks.
struct GemmCfg {
    int wn, wk;
};

// (WN, WK) = (8, 1), (4, 2) or (2, 4).  The widest tile that still gives three
// quarters of the CUs a workgroup (measured: at 512 x 14336 x 4096, 224
// workgroups of (8, 1) beat 448 of (4, 2) by 10 %), else the one with the most
// workgroups (WK must divide the groups per row).
inline GemmCfg choose_gemm(int M, int N, int K, int cus)
{
    const int G = K / 64;
    const int64_t tm = ((int64_t)M + kGemmTileM - 1) / kGemmTileM;
    const int opts[3][2] = {{8, 1}, {4, 2}, {2, 4}};
    GemmCfg best{8, 1};
    int64_t best_t = -1;
    for (const auto& o : opts) {
        if (G % o[1] != 0) continue;
        const int64_t t = (((int64_t)N + 64 * o[0] - 1) / (64 * o[0])) * tm;
        if (4 * t >= 3 * (int64_t)cus) return GemmCfg{o[0], o[1]};
        if (t > best_t) {
            best_t = t;
            best = GemmCfg{o[0], o[1]};
        }
    }
    return best;
}

// Workgroups per tile that split its groups when the tiles alone leave more
// than a quarter of the CUs idle (1024-row matrices): the smallest ks = 2..8
// that fills three quarters of the CUs with at least 2 groups per wavefront
// chunk (ks WK must divide the groups), else the largest such ks; 1 when
// none fits.  Each tile's ks partial products are summed by a second kernel
// in a fixed order.
inline int gemm_ksplit(int M, int N, int K, GemmCfg g, int cus)
{
    const int G = K / 64;
    const int64_t T = (((int64_t)N + 64 * g.wn - 1) / (64 * g.wn)) * (((int64_t)M + kGemmTileM - 1) / kGemmTileM);
    if (4 * T >= 3 * (int64_t)cus) return 1;
    int best = 1;
    for (int ks = 2; ks <= 8; ++ks) {
        if (G % (g.wk * ks) != 0 || G / (g.wk * ks) < 2) continue;
        best = ks;
        if (4 * T * ks >= 3 * (int64_t)cus) break;
    }
    return best;
}

// Bytes of the partial products when the tiles are split ks ways.
inline size_t gemm_part_bytes(int M, int N, int ks)
{
    return ks > 1 ? ((size_t)ks * M * N * 4 + 255) / 256 * 256 : 0;
}

// Workspace that lets a prompt GEMM use its K split on a full 256-CU gfx950:
// the base (x operands, pieces) plus the partial products.  A workspace of at
// least the base is accepted; the split is used only where the partials fit.
inline size_t gemm_workspace_bytes(int bits, int M, int N, int K)
{
    const GemmCfg g = choose_gemm(M, N, K, 256);
    return gemm_workspace_base(bits, M, K) + gemm_part_bytes(M, N, gemm_ksplit(M, N, K, g, 256));
}

// Affine prompt GEMM, BITS = 2..8 (affine_gemm_b*.hip): the pre-pass over x,
// then the main kernel.
template <int BITS>
hipError_t launch_affine_gemm(const GemmArgs& a, hipStream_t s);

// bits: 0 = dense bf16, 2..8 = affine width.
LaunchCfg choose_config(int bits, bool swiglu, int M, int N, int K);
hipError_t launch_proj(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_unpack(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, hipStream_t s);

}  // namespace aqg
