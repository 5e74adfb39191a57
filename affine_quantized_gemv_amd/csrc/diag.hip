// Stream-read probe for the measurement harness: reads `bytes` bytes once with
// the access pattern of the weight streams (16-byte buffer loads, whole
// 128-byte lines per instruction, non-temporal) and nothing else, so its
// time over a range of sizes gives this machine's read ceiling t0 + bytes/BW
// against which the projections are reported.
#include "aqgemv.h"
#include "host_query.h"
#include "piece_kernel.h"

namespace aqg {
namespace detail {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;         // 16-byte loads in flight per lane

__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const char* __restrict__ src, int64_t bytes,
                                                                   float* __restrict__ sink)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t nthreads = (int64_t)gridDim.x * kReadThreads;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * kReadThreads + wave * 64;   // the wavefront's first thread
    const int64_t t = t0 + (threadIdx.x & 63);
    const int64_t pieces = bytes / 16;
    uint32_t acc = 0;
    // chunks of kReadUnroll consecutive sweeps of the grid: each load
    // instruction of a wavefront covers 1 KB of consecutive bytes
    for (int64_t base = 0; base < pieces; base += nthreads * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t p = base + (int64_t)u * nthreads + t;
            // a wave-uniform 1 GB window (the descriptor's offset is 32 bits;
            // a wavefront's 1 KB never leaves the window's 2 GB range)
            const int64_t win = ((base + (int64_t)u * nthreads + t0) * 16) & ~(int64_t)0x3FFFFFFF;
            const int64_t off = p < pieces ? p * 16 : win;
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(src + win, bytes - win);
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(off - win), 0, kLoadNT));
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = 1.0f;      // keeps the loads; (almost) never stores
}

}  // namespace
}  // namespace detail
}  // namespace aqg

extern "C" int aqg_stream_read(const void* src, size_t bytes, float* sink, void* stream)
{
    if (!src || !sink || bytes < 16) return AQG_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0) return AQG_ERR_ALIGNMENT;
    int cus = 0;
    if (aqg::detail::device_cus(cus) != hipSuccess) {
        (void)hipGetLastError();
        return AQG_ERR_DEVICE;
    }
    // eight 4-wavefront workgroups per CU (~32 KB in flight per CU)
    const int64_t want = (int64_t)(bytes / 16 + aqg::detail::kReadThreads - 1) / aqg::detail::kReadThreads;
    int64_t blocks = (int64_t)cus * 8;
    if (blocks > want) blocks = want > 0 ? want : 1;
    hipLaunchKernelGGL(aqg::detail::stream_read_kernel, dim3((unsigned)blocks), dim3(aqg::detail::kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const char*>(src), (int64_t)bytes, sink);
    if (hipGetLastError() != hipSuccess) return AQG_ERR_LAUNCH;
    return AQG_OK;
}
