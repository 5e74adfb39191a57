// Host-side interface between the C ABI (abi.hip) and the kernels
// (kernels.hip).  Not installed; not part of the public ABI.
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
    int lpr_log2;            // log2 of lanes that share one weight row
    int out_f32;             // 1: store fp32, 0: store bf16 (RNE)
};

// Launch geometry chosen for a call.
struct LaunchCfg {
    int MT;         // padded M (1, 2, 4, 8, 16, 32)
    int R;          // rows per lane (1 or 2)
    int lpr_log2;   // lanes per weight row = 2^lpr_log2 (<= 16)
    int KT;         // K-tile in elements
    int nwaves;     // waves per workgroup
    int blocks;     // workgroups
    size_t lds;     // dynamic LDS bytes
};

// Per-width launchers, each instantiated in its own translation unit
// (proj_b*.hip) so the kernels compile in parallel.
template <int BITS, bool SWIGLU>
hipError_t launch_bits(const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

// bits: 0 = dense bf16, 2..8 = affine width.
LaunchCfg choose_valu(int bits, bool swiglu, int M, int N, int K);
hipError_t launch_valu(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_unpack(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, hipStream_t s);

}  // namespace aqg
