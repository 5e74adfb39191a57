// Host-side interface between the C ABI (abi.hip) and the kernels
// (kernels.hip, proj_b*.hip, mfma_*.hip).  Not installed; not part of the
// public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aqg {

// Arguments of one projection launch.  Pointers are device pointers.
struct ProjArgs {
    const uint16_t* x;       // bf16 [M][K]
    const void* w0;          // dense W, affine Wq words, or SwiGLU Wg
    const void* w1;          // SwiGLU Wu (else null)
    const uint16_t* scales;  // affine: bf16 [N][K/64]
    const uint16_t* biases;  // affine: bf16 [N][K/64]
    void* y;                 // bf16 or f32 [M][N]
    int M, N, K;
    int KT;                  // K elements staged in LDS per tile
    int lpr_log2;            // VALU/stream paths: log2 of lanes that share one weight row
    int ksplit_log2;         // MFMA path: log2 of wavefronts splitting K per row group
    int out_f32;             // 1: store fp32, 0: store bf16 (RNE)
    int64_t tpw;             // stream path: row tiles per super-tile
    int64_t tmax;            // stream path: most row tiles any wavefront finishes
};

enum Path { PATH_VALU = 0, PATH_MFMA = 1, PATH_STREAM = 2, PATH_PIECE = 3, PATH_MFMA_STREAM = 4, PATH_MFMA_SPLIT = 5, PATH_AFFINE_MFMA = 6,
            PATH_MFMA_TILE = 7, PATH_AFFINE_TILE = 8, PATH_AFFINE_SPLIT = 9 };

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
// 16-row tile, BITS = 2, 4 or 8 (affine_split.hip).
template <int BITS>
hipError_t launch_affine_split(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// Affine matrix-core launcher, BITS = 2, 4 or 8 (affine_mfma*.hip).
template <int BITS>
hipError_t launch_affine_mfma(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// bits: 0 = dense bf16, 2..8 = affine width.
LaunchCfg choose_config(int bits, bool swiglu, int M, int N, int K);
hipError_t launch_proj(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_unpack(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, hipStream_t s);

}  // namespace aqg
