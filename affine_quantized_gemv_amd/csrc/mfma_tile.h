// Persistent matrix-core kernel for large-N dense projections at M = 3..32
// (M padded to 16 or 32) with K = 512, 1024, 1536 or 2048, on gfx950.
//
// y^T[N, M] = W[N, K] . x^T[K, M] with v_mfma_f32_16x16x32_bf16 (operand
// layouts as in mfma_kernel.h).  A row tile is 16 rows of W, i.e. 32 K
// consecutive bytes of HBM.  Where the per-wavefront stream (mfma_stream.h)
// has every wavefront walk the 16 rows of its own tile side by side, here a
// workgroup fetches whole tiles in address order:
//
//   * Each of the 8 wavefronts copies K/256 consecutive 1 KB pieces of the
//     tile straight into LDS (buffer loads with an LDS destination, 16 bytes
//     per lane), so every load instruction reads 1 KB of consecutive bytes
//     and the workgroup sweeps the matrix front to back: the access order
//     that measured fastest for a plain read of a large matrix on this chip
//     (~6.8 TB/s, against ~6.0 TB/s when each instruction covers 8 rows).
//     Rows sit in LDS with a 16-byte pad, so the MFMA operand reads that
//     follow are free of bank conflicts.
//   * NBUF tile buffers form a ring.  As soon as every wavefront has read
//     its operands from a buffer, the tile NBUF places ahead is issued into
//     it, so up to NBUF tiles are in flight.  The copies are written as
//     inline assembly: the compiler's wait insertion cannot tell a copy into
//     one buffer from an operand read of another and would otherwise wait
//     for every copy in flight before each read.  The kernel waits itself,
//     with counts that leave exactly the younger copies and stores in flight.
//   * Wavefront w owns k in [w K/8, (w+1) K/8) of every tile and keeps the
//     x^T B operands of that range in registers for the whole launch.  Per
//     tile it reads its A operands from LDS and runs K/256 MFMAs per
//     16-column block; the 8 partial 16 x MT tiles are summed through LDS in
//     wavefront order 0, 1, ..., 7 (fixed: results do not depend on M).
//   * Each thread sums one output of the tile over the 8 partials and stores
//     it with one buffer store (dropped by the hardware when out of range),
//     so every wavefront issues the same, known number of memory operations
//     per step and the wait for the next tile can leave exactly the younger
//     ones outstanding.
//   * The two barriers of a step are plain s_barrier with explicit waits:
//     __syncthreads() would also wait for every tile still in flight.
//   * Consecutive tiles are processed by workgroups of the same XCD, so the
//     output lines they share are completed in one L2.
//
// Shapes: AstrAI decode_linear_benchmark.md (commit message; the LM head and
// M = 1..32 decode shapes).
#pragma once

#include "argmax.h"
#include "mfma_kernel.h"
#include "piece_kernel.h"

namespace aqg {
namespace detail {

constexpr int kMfmaTileWaves = 8;
constexpr int kMfmaTileThreads = 64 * kMfmaTileWaves;

template <int MT, int KSW, int NBUF, int NW = kMfmaTileWaves>
struct MfmaTileLayout {
    static constexpr int K = 256 * KSW;           // k per row
    static constexpr int NT = 64 * NW;            // threads per workgroup
    static constexpr int KSTEPS = K / 32 / NW;    // k-steps per wavefront
    static constexpr int ROW = 2 * K;             // bytes per weight row
    static constexpr int RS = ROW + 16;           // LDS row stride (bank pad)
    static constexpr int TILE = 16 * RS;          // LDS bytes per tile buffer
    static constexpr int CPW = 8 * KSW / NW;      // 1 KB pieces per wavefront per tile
    static constexpr int CPR = ROW / 1024;        // 1 KB pieces per row
    static constexpr int NB = MT / 16;            // 16-column blocks of x^T
    static constexpr int PW = NB * 4 * 65;        // floats per wavefront partial (65: bank pad)
    static constexpr int PART = NW * PW * 4;
    static constexpr size_t LDS = (size_t)NBUF * TILE + PART;
    static_assert(ROW % 1024 == 0, "pieces never straddle rows");
    static_assert(16 * ROW / 1024 == NW * CPW, "pieces split evenly over the wavefronts");
    static_assert(KSTEPS * 32 * NW == K, "k-steps split evenly over the wavefronts");
};

// Distinct LDS objects: buffer I of BYTES bytes.
template <int I, int BYTES>
__device__ __forceinline__ char* mfma_tile_lds()
{
    __shared__ __attribute__((aligned(16))) char b[BYTES];
    return b;
}

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// Buffer descriptor words for `bytes` bytes at p (raw buffer, stride 0).
__device__ __forceinline__ u32x4v_t buffer_words(const void* p, int64_t bytes)
{
    const uint64_t base = reinterpret_cast<uint64_t>(p);
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7FFFFFF0 ? 0x7FFFFFF0u : (uint32_t)bytes);
    return u32x4v_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, n, (uint32_t)kBufferFlags};
}

// 16 bytes per lane from buffer offset soff + voff into LDS at lds + 16 lane
// (non-temporal).  The data goes to LDS only; no register is written.
__device__ __forceinline__ void copy_1k_to_lds(u32x4v_t rs, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) and lgkmcnt(0), expcnt not waited.
__host__ __device__ constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }
__host__ __device__ constexpr int waitcnt_lgkm0() { return 0x3F | (3 << 14) | 0x70; }

__device__ __forceinline__ void barrier_only()
{
    // a barrier with no implied wait for loads in flight; the memory clobber
    // keeps the compiler from moving LDS accesses across it
    asm volatile("s_barrier" ::: "memory");
}

template <int MT, int KSW, int NBUF, int NW = kMfmaTileWaves>
__global__ void __launch_bounds__(64 * NW) mfma_tile_kernel(ProjArgs a)
{
    using L = MfmaTileLayout<MT, KSW, NBUF, NW>;
    constexpr int NB = L::NB;
    static_assert(NBUF >= 1 && NBUF <= 4, "ring of 1..4 tiles");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane >> 4;             // k sub-block (A, B) / row quad (D)
    const int r = lane & 15;             // A row / B and D column
    const int64_t T = ((int64_t)a.N + 15) / 16;
    // Tiles are dealt round-robin over the workgroups taken in XCD-major
    // order (workgroup b runs on XCD b % 8), so consecutive tiles run on one
    // XCD: the 32-byte pieces that neighbouring tiles write into each 128-byte
    // output line meet in that XCD's L2 instead of leaving several L2s as
    // partial lines (measured 60 -> 54 us on the 100000 x 1536 LM head at
    // M = 32).
    const int64_t G8 = gridDim.x / 8;
    const int64_t first = (gridDim.x % 8 == 0) ? (int64_t)(blockIdx.x % 8) * G8 + blockIdx.x / 8 : blockIdx.x;
    const int64_t stride = gridDim.x;
    if (first >= T) {
        if (a.amx && threadIdx.x < kArgmaxRows)
            amx_store(a.amx, a.amx_slots, blockIdx.x, threadIdx.x, amx_neutral_value(), kAmxNoIndex);
        return;
    }
    const int64_t ntile = (T - 1 - first) / stride + 1;   // tiles of this workgroup (uniform)

    float* part = reinterpret_cast<float*>(mfma_tile_lds<NBUF, L::PART>());

    // copy local tile j into buffer B: 1 KB pieces wave*CPW .. + CPW - 1
    auto issue = [&](int64_t j, auto Bc) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
        const int64_t n0 = (first + j * stride) * 16;
        const u32x4v_t rs = buffer_words(static_cast<const char*>(a.w0) + n0 * L::ROW, (a.N - n0) * L::ROW);
        const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)mfma_tile_lds<B, L::TILE>();
#pragma unroll
        for (int q = 0; q < L::CPW; ++q) {
            const int piece = wave * L::CPW + q;
            const int row = piece / L::CPR, col = piece - row * L::CPR;
            // the piece's offset in the vector offset, which the range check covers
            copy_1k_to_lds(rs, dst + row * L::RS + col * 1024, (uint32_t)(lane * 16 + piece * 1024), 0);
        }
    };

    // The first tile, then this wavefront's x^T operands, then the rest of
    // the ring: the wait for x (which the compiler places as a wait for
    // every load in flight) covers one tile rather than the whole ring, and
    // the first tile's arithmetic overlaps the others' copies.
    issue(0, Int<0>{});
    u32x4_t xr[L::KSTEPS][NB];
    const int kw = wave * (L::K / NW);
#pragma unroll
    for (int s = 0; s < L::KSTEPS; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int m = 16 * b + r;
            xr[s][b] = u32x4_t{0u, 0u, 0u, 0u};
            if (m < a.M)
                xr[s][b] = *reinterpret_cast<const u32x4_t*>(a.x + (size_t)m * L::K + kw + 32 * s + 8 * c);
        }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    static_for<1, NBUF>([&](auto Bc) __attribute__((always_inline)) {
        if (decltype(Bc)::value < ntile) issue(decltype(Bc)::value, Bc);
    });
    barrier_only();   // tile 0 is in LDS: every wavefront waited for its copies

    // reducer role of this thread: output (m, n) of each tile.  Every lane
    // issues exactly one buffer store per tile (lanes without an output
    // store out of range, which the hardware drops), so each wavefront issues
    // a known number of memory operations per step.
    const int t = threadIdx.x;
    const bool red = t < 16 * MT;
    const int om = t >> 4, on = t & 15;
    const int pidx = ((om >> 4) * 4 + (on & 3)) * 65 + (on >> 2) * 16 + (om & 15);
    const int esz = a.out_f32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ry = tile_rsrc(a.y, (int64_t)a.M * a.N * esz);
    constexpr uint32_t kDrop = 0x80000000u;   // beyond any output range
    // row argmax (a.amx): the thread's running maximum of its outputs, all of
    // row om; the store is still issued, out of range, so that every
    // wavefront's count of memory operations per step stays the same
    float amx_v = amx_neutral_value();
    int amx_i = kAmxNoIndex;

    auto step = [&](int64_t j, auto Bc) __attribute__((always_inline)) {
        constexpr int B = decltype(Bc)::value;
        // this wavefront's k range of tile j (buffer B)
        const char* src = mfma_tile_lds<B, L::TILE>() + r * L::RS + (kw + 8 * c) * 2;
        f32x4_t acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < L::KSTEPS; ++s) {
            const u32x4_t A = *reinterpret_cast<const u32x4_t*>(src + 64 * s);
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = mfma16x16x32(A, xr[s][b], acc[b]);
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

        const float* p = part + (red ? pidx : 0);
        float v = p[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += p[w * L::PW];
        const int64_t n = (first + j * stride) * 16 + on;
        const bool live = red && om < a.M && n < a.N;
        uint32_t off = live ? (uint32_t)(((int64_t)om * a.N + n) * esz) : kDrop;
        if (a.amx) {
            if (live) amx_take(amx_v, amx_i, v, (int)n);
            off = kDrop;
        }
        if (a.out_f32) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), ry, off, 0, 0);

        // Tile j + 1 must be in LDS before the next step.  When it was issued
        // by step j + 1 - NBUF, the operations issued after its copy are that
        // step's store, then per step since: the copy of a tile (CPW pieces,
        // if the tile exists) and one store.  Those may stay in flight: nd
        // copies (tiles j+2 .. j+NBUF that exist) and NBUF stores.  When it
        // was issued in the prologue (j = B < NBUF - 1), the operations after
        // its copy are the prologue's later tiles and, per step 0..B, one
        // tile's copy (if the tile exists) and one store.
        const bool from_step = j + 1 >= NBUF;
        if (from_step) {
            const int64_t nd64 = ntile - 2 - j;
            const int nd = nd64 < 0 ? 0 : (nd64 > NBUF - 1 ? NBUF - 1 : (int)nd64);
            static_for<0, NBUF>([&](auto Dc) __attribute__((always_inline)) {
                constexpr int D = decltype(Dc)::value;
                if (nd == D) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(D * L::CPW + NBUF));
            });
        } else {
            const int64_t lim = ntile < NBUF ? ntile : NBUF;
            const int64_t np = lim - (B + 2) > 0 ? lim - (B + 2) : 0;                    // later prologue tiles
            const int64_t ns = ntile - NBUF > 0 ? (ntile - NBUF < B + 1 ? ntile - NBUF : B + 1) : 0;   // tiles issued by steps 0..B
            const int q = (int)(np + ns);
            static_for<0, NBUF>([&](auto Qc) __attribute__((always_inline)) {
                constexpr int Q = decltype(Qc)::value;
                if (q == Q) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(Q * L::CPW + B + 1));
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
    if (a.amx) {
        // the 16 threads of row om are one 16-lane row of a wavefront: the
        // DPP row tree combines them
        amx_row(amx_v, amx_i);
        if (on == 0 && om < kArgmaxRows) amx_store(a.amx, a.amx_slots, blockIdx.x, om, amx_v, amx_i);
    }
}

// Tile buffers for a K: enough that NBUF - 1 tiles (~48 KB or more) are in
// flight, within one CU's LDS at M = 32.
inline int mfma_tile_nbuf(int K)
{
    switch (K) {
        case 512: return 4;
        case 1024: return 3;
        case 1536: return 2;
        case 2048: return 2;
        default: return 0;
    }
}

// Large N (>= 2048 row tiles), K with a tile ring, and outputs addressable by
// one 32-bit buffer offset at any M (32 N 4 bytes below 2 GB).  Depends on
// (N, K) only, so every M the path serves computes each output the same way.
inline bool mfma_tile_supported(int N, int K, bool swiglu)
{
    return !swiglu && mfma_tile_nbuf(K) != 0 && ((int64_t)N + 15) / 16 >= 2048 &&
           (int64_t)32 * N * 4 < 0x7FFFFFF0;
}

template <int MT, int KSW, int NBUF, int NW = kMfmaTileWaves>
hipError_t launch_mfma_tile_one(const ProjArgs& a, hipStream_t s)
{
    static_assert(MfmaTileLayout<MT, KSW, NBUF, NW>::LDS <= 160 * 1024, "fits one CU's LDS");
    const void* fn = reinterpret_cast<const void*>(&mfma_tile_kernel<MT, KSW, NBUF, NW>);
    int cus = 0, bpc = 0;
    hipError_t e = device_cus(cus);
    if (e == hipSuccess) e = occupancy(bpc, fn, 64 * NW, 0);
    if (e != hipSuccess) return e;
    if (bpc < 1) bpc = 1;
    const int64_t T = ((int64_t)a.N + 15) / 16;
    int64_t blocks = (int64_t)bpc * cus;
    if (blocks > T) blocks = T;
    if (a.amx && blocks > a.amx_slots) return hipErrorInvalidValue;   // one partial per workgroup
    if (a.amx_producers) *a.amx_producers = blocks;
    hipLaunchKernelGGL((mfma_tile_kernel<MT, KSW, NBUF, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mfma_tile_mt(const ProjArgs& a, hipStream_t s)
{
    switch (a.K) {
        case 512: return launch_mfma_tile_one<MT, 2, 4>(a, s);
        case 1024: return launch_mfma_tile_one<MT, 4, 3>(a, s);
        case 1536: return launch_mfma_tile_one<MT, 6, 2>(a, s);
        case 2048: return launch_mfma_tile_one<MT, 8, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

inline hipError_t launch_mfma_tile_impl(const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (a.w1 != nullptr || !mfma_tile_supported(a.N, a.K, false)) return hipErrorInvalidValue;
    switch (c.MT) {
        case 16: return launch_mfma_tile_mt<16>(a, s);
        case 32: return launch_mfma_tile_mt<32>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace detail
}  // namespace aqg
