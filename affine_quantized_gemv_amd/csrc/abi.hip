// C ABI of libaqgemv.so (declared in include/aqgemv.h): argument validation
// on the host, a cached per-device gfx950 check, geometry choice and launch.
//
// The refusal rules follow the pages' lessons: unsupported widths, group sizes
// and shapes are refused rather than silently handled (TensorFold PR #849,
// "Groups other than 64, and non-affine modes, are still refused"; sizes must
// be positive, same PR, config-parse fix); a launch is always checked so an
// output is never left unwritten without an error (FreeToken-Kai
// docs/turing.md, sgl_kernel section: unchecked launches left torch.empty
// outputs uninitialised).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "aqgemv.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch[kMaxDevices];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return AQG_ERR_DEVICE;
    }
    int state = g_arch[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return AQG_ERR_DEVICE;
        }
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? AQG_OK : AQG_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bn && b0 < a0 + an;
}

int check_common(const void* x, const void* y, int M, int N, int K, int out_dtype)
{
    if (!x || !y) return AQG_ERR_INVALID_ARG;
    if (M <= 0 || N <= 0 || K <= 0) return AQG_ERR_INVALID_ARG;
    if (out_dtype != AQG_OUT_BF16 && out_dtype != AQG_OUT_F32) return AQG_ERR_INVALID_ARG;
    if (M > 32) return AQG_ERR_UNSUPPORTED;
    if (!aligned(x, 16)) return AQG_ERR_ALIGNMENT;
    if (!aligned(y, out_dtype == AQG_OUT_F32 ? 4 : 2)) return AQG_ERR_ALIGNMENT;
    return AQG_OK;
}

size_t out_bytes(int M, int N, int out_dtype)
{
    return (size_t)M * (size_t)N * (out_dtype == AQG_OUT_F32 ? 4 : 2);
}

int finish(hipError_t e)
{
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return AQG_ERR_LAUNCH;
    }
    return AQG_OK;
}

int run_projection(int bits, bool swiglu, const void* x, const void* w0, const void* w1,
                   const void* scales, const void* biases, void* y, int M, int N, int K,
                   int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_common(x, y, M, N, K, out_dtype);
    if (st != AQG_OK) return st;
    if (!w0 || (swiglu && !w1) || (bits && (!scales || !biases))) return AQG_ERR_INVALID_ARG;
    if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return AQG_ERR_UNSUPPORTED;
    if (!aligned(w0, 16) || (w1 && !aligned(w1, 16))) return AQG_ERR_ALIGNMENT;
    // the matrix-core kernels read scales and biases in 4- to 16-byte pieces
    if (bits && (!aligned(scales, 4) || !aligned(biases, 4))) return AQG_ERR_ALIGNMENT;
    const int kind = swiglu ? AQG_KIND_SWIGLU : bits;
    if (workspace_bytes < aqg_workspace_bytes(kind, M, N, K)) return AQG_ERR_INVALID_ARG;
    (void)workspace;

    const size_t ybytes = out_bytes(M, N, out_dtype);
    const size_t xbytes = (size_t)M * K * 2;
    const size_t wbytes = bits ? (size_t)N * K / 8 * bits : (size_t)N * K * 2;
    const size_t gbytes = (size_t)N * (K / 64) * 2;
    if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, w0, wbytes) ||
        (swiglu && overlap(y, ybytes, w1, wbytes)) ||
        (bits && (overlap(y, ybytes, scales, gbytes) || overlap(y, ybytes, biases, gbytes))))
        return AQG_ERR_INVALID_ARG;

    st = check_device();
    if (st != AQG_OK) return st;

    const aqg::LaunchCfg cfg = aqg::choose_config(bits, swiglu, M, N, K);
    aqg::ProjArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w0 = w0;
    a.w1 = w1;
    a.scales = static_cast<const uint16_t*>(scales);
    a.biases = static_cast<const uint16_t*>(biases);
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.KT = cfg.KT;
    a.lpr_log2 = cfg.lpr_log2;
    a.ksplit_log2 = cfg.ksplit_log2;
    a.tpw = cfg.tpw;
    a.out_f32 = out_dtype == AQG_OUT_F32;
    return finish(aqg::launch_proj(bits, swiglu, a, cfg, static_cast<hipStream_t>(stream)));
}

int run_affine(int bits, const void* x, const uint32_t* Wq, const void* scales, const void* biases,
               void* y, int M, int N, int K, int out_dtype, void* ws, size_t wsb, void* stream)
{
    return run_projection(bits, false, x, Wq, nullptr, scales, biases, y, M, N, K, out_dtype, ws, wsb,
                          stream);
}

}  // namespace

extern "C" {

int aqg_abi_version(void) { return AQG_ABI_VERSION; }

const char* aqg_status_string(int status)
{
    switch (status) {
        case AQG_OK: return "AQG_OK: success";
        case AQG_ERR_INVALID_ARG: return "AQG_ERR_INVALID_ARG: null pointer, non-positive size, bad out_dtype, "
                                         "short workspace or overlapping output";
        case AQG_ERR_UNSUPPORTED: return "AQG_ERR_UNSUPPORTED: M > 32, K not a multiple of 8 (dense) or 64 "
                                         "(affine), or bits outside 2..8";
        case AQG_ERR_ALIGNMENT: return "AQG_ERR_ALIGNMENT: x and W/Wq must be 16-byte aligned, scales and "
                                       "biases 4-byte aligned, other arrays aligned to their element size";
        case AQG_ERR_LAUNCH: return "AQG_ERR_LAUNCH: the kernel launch failed";
        case AQG_ERR_DEVICE: return "AQG_ERR_DEVICE: no current HIP device, or it is not gfx950";
        default: return "unknown aqg status";
    }
}

size_t aqg_workspace_bytes(int kind, int M, int N, int K)
{
    (void)kind; (void)M; (void)N; (void)K;
    return 0;  // no variant uses split-K partials yet
}

int aqg_gemv_bf16(const void* x, const void* W, void* y, int M, int N, int K, int out_dtype,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    return run_projection(0, false, x, W, nullptr, nullptr, nullptr, y, M, N, K, out_dtype, workspace,
                          workspace_bytes, stream);
}

int aqg_swiglu_bf16(const void* x, const void* Wg, const void* Wu, void* out, int M, int N, int K,
                    int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return run_projection(0, true, x, Wg, Wu, nullptr, nullptr, out, M, N, K, out_dtype, workspace,
                          workspace_bytes, stream);
}

#define AQG_AFFINE_ENTRY(B)                                                                          \
    int aqg_gemv_affine_q##B(const void* x, const uint32_t* Wq, const void* scales, const void* biases, \
                             void* y, int M, int N, int K, int out_dtype, void* workspace,          \
                             size_t workspace_bytes, void* stream)                                  \
    {                                                                                                \
        return run_affine(B, x, Wq, scales, biases, y, M, N, K, out_dtype, workspace, workspace_bytes, \
                          stream);                                                                   \
    }
AQG_AFFINE_ENTRY(2)
AQG_AFFINE_ENTRY(3)
AQG_AFFINE_ENTRY(4)
AQG_AFFINE_ENTRY(5)
AQG_AFFINE_ENTRY(6)
AQG_AFFINE_ENTRY(7)
AQG_AFFINE_ENTRY(8)
#undef AQG_AFFINE_ENTRY

int aqg_unpack_codes(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, void* stream)
{
    if (!Wq || !codes || N <= 0 || K <= 0) return AQG_ERR_INVALID_ARG;
    if (bits < 2 || bits > 8 || K % 64 != 0) return AQG_ERR_UNSUPPORTED;
    if (!aligned(Wq, 16) || !aligned(codes, 16)) return AQG_ERR_ALIGNMENT;
    if (overlap(codes, (size_t)N * K, Wq, (size_t)N * K / 8 * bits)) return AQG_ERR_INVALID_ARG;
    int st = check_device();
    if (st != AQG_OK) return st;
    return finish(aqg::launch_unpack(bits, Wq, codes, N, K, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
