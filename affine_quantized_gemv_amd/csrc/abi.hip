// C ABI of libaqgemv.so (declared in include/aqgemv.h): argument validation
// on the host, a cached per-device gfx950 check, geometry choice and launch.
//
// The refusal rules follow the pages' lessons: unsupported widths, group sizes
// and shapes are refused rather than silently handled (TensorFold PR #849,
// "What this changes": only the affine mode with groups of 64 is accepted;
// sizes must be positive, same PR, config-parse fix); a launch is always
// checked so an output is never left unwritten without an error
// (FreeToken-Kai docs/turing.md, sgl_kernel section: a launch whose failure
// went unchecked left its outputs uninitialised).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "aqgemv.h"
#include "host_query.h"
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
                   const void* scales, const void* biases, const void* scales1, const void* biases1, void* y,
                   int M, int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_common(x, y, M, N, K, out_dtype);
    if (st != AQG_OK) return st;
    const bool two = swiglu && bits;     // affine SwiGLU: the up matrix has its own scales and biases
    if (!w0 || (swiglu && !w1) || (bits && (!scales || !biases)) || (two && (!scales1 || !biases1)))
        return AQG_ERR_INVALID_ARG;
    if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return AQG_ERR_UNSUPPORTED;
    if (!aligned(w0, 16) || (w1 && !aligned(w1, 16))) return AQG_ERR_ALIGNMENT;
    // the matrix-core kernels read scales and biases in 4- to 16-byte pieces
    if (bits && (!aligned(scales, 4) || !aligned(biases, 4))) return AQG_ERR_ALIGNMENT;
    if (two && (!aligned(scales1, 4) || !aligned(biases1, 4))) return AQG_ERR_ALIGNMENT;
    const int kind = swiglu ? (bits ? AQG_KIND_SWIGLU_AFFINE + bits : AQG_KIND_SWIGLU) : bits;
    if (workspace_bytes < aqg_workspace_bytes(kind, M, N, K)) return AQG_ERR_INVALID_ARG;
    (void)workspace;

    const size_t ybytes = out_bytes(M, N, out_dtype);
    const size_t xbytes = (size_t)M * K * 2;
    const size_t wbytes = bits ? (size_t)N * K / 8 * bits : (size_t)N * K * 2;
    const size_t gbytes = (size_t)N * (K / 64) * 2;
    if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, w0, wbytes) ||
        (swiglu && overlap(y, ybytes, w1, wbytes)) ||
        (bits && (overlap(y, ybytes, scales, gbytes) || overlap(y, ybytes, biases, gbytes))) ||
        (two && (overlap(y, ybytes, scales1, gbytes) || overlap(y, ybytes, biases1, gbytes))))
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
    a.scales1 = static_cast<const uint16_t*>(scales1);
    a.biases1 = static_cast<const uint16_t*>(biases1);
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
    return run_projection(bits, false, x, Wq, nullptr, scales, biases, nullptr, nullptr, y, M, N, K, out_dtype,
                          ws, wsb, stream);
}

// ------------------------------------------------ prompt GEMM

hipError_t launch_gemm_bits(int bits, const aqg::GemmArgs& a, hipStream_t s)
{
    switch (bits) {
        case 2: return aqg::launch_affine_gemm<2>(a, s);
        case 3: return aqg::launch_affine_gemm<3>(a, s);
        case 4: return aqg::launch_affine_gemm<4>(a, s);
        case 5: return aqg::launch_affine_gemm<5>(a, s);
        case 6: return aqg::launch_affine_gemm<6>(a, s);
        case 7: return aqg::launch_affine_gemm<7>(a, s);
        case 8: return aqg::launch_affine_gemm<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

int run_gemm(int bits, const void* x, const uint32_t* Wq, const void* scales, const void* biases, void* y,
             int M, int N, int K, int out_dtype, void* ws, size_t wsb, void* stream)
{
    if (!x || !y || !Wq || !scales || !biases) return AQG_ERR_INVALID_ARG;
    if (M <= 0 || N <= 0 || K <= 0) return AQG_ERR_INVALID_ARG;
    if (out_dtype != AQG_OUT_BF16 && out_dtype != AQG_OUT_F32) return AQG_ERR_INVALID_ARG;
    if (M > AQG_GEMM_MAX_M || K % 64 != 0) return AQG_ERR_UNSUPPORTED;
    const size_t need = aqg::gemm_workspace_base(bits, M, K);
    if (!ws || wsb < need) return AQG_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(Wq, 16) || !aligned(ws, 16)) return AQG_ERR_ALIGNMENT;
    if (!aligned(scales, 4) || !aligned(biases, 4)) return AQG_ERR_ALIGNMENT;
    if (!aligned(y, out_dtype == AQG_OUT_F32 ? 4 : 2)) return AQG_ERR_ALIGNMENT;
    const size_t ybytes = out_bytes(M, N, out_dtype);
    const size_t xbytes = (size_t)M * K * 2;
    const size_t wbytes = (size_t)N * K / 8 * bits;
    const size_t gbytes = (size_t)N * (K / 64) * 2;
    const void* in[4] = {x, Wq, scales, biases};
    const size_t inb[4] = {xbytes, wbytes, gbytes, gbytes};
    for (int i = 0; i < 4; ++i)
        if (overlap(y, ybytes, in[i], inb[i]) || overlap(ws, need, in[i], inb[i])) return AQG_ERR_INVALID_ARG;
    if (overlap(ws, need, y, ybytes)) return AQG_ERR_INVALID_ARG;
    int st = check_device();
    if (st != AQG_OK) return st;
    // tiling and K split for this device; the split only where the workspace
    // also holds its partial products (and they overlap no argument)
    int cus = 256;
    if (aqg::detail::device_cus(cus) != hipSuccess) cus = 256;
    const aqg::GemmCfg g = aqg::choose_gemm(M, N, K, cus);
    int ks = aqg::gemm_ksplit(M, N, K, g, cus);
    const size_t pb = aqg::gemm_part_bytes(M, N, ks);
    if (ks > 1 && wsb < need + pb) ks = 1;
    if (ks > 1) {
        const void* part = static_cast<char*>(ws) + need;
        for (int i = 0; i < 4; ++i)
            if (overlap(part, pb, in[i], inb[i])) return AQG_ERR_INVALID_ARG;
        if (overlap(part, pb, y, ybytes)) return AQG_ERR_INVALID_ARG;
    }

    aqg::GemmArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.wq = Wq;
    a.scales = static_cast<const uint16_t*>(scales);
    a.biases = static_cast<const uint16_t*>(biases);
    a.y = y;
    a.xp = static_cast<uint16_t*>(ws);
    a.pieces = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + aqg::gemm_pieces_offset(M, K));
    a.M = M;
    a.N = N;
    a.K = K;
    a.G = K / 64;
    a.Gp = (a.G + 31) / 32 * 32;
    a.Mp = (M + aqg::kGemmTileM - 1) / aqg::kGemmTileM * aqg::kGemmTileM;
    a.out_f32 = out_dtype == AQG_OUT_F32;
    a.wn = g.wn;
    a.ks = ks;
    a.part = ks > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + need) : nullptr;
    return finish(launch_gemm_bits(bits, a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ multi-projection launch

// The kernels that take a segment table (several projections of one x in
// one launch): one row tile per workgroup, or a persistent walk over tiles
// that looks up each tile's projection.
bool multi_fused(const aqg::LaunchCfg& c)
{
    return c.path == aqg::PATH_PIECE || c.path == aqg::PATH_MFMA_SPLIT || c.path == aqg::PATH_AFFINE_SPLIT;
}

int run_multi(int bits, const void* x, int P, const void* const* W, const void* const* scales,
              const void* const* biases, void* const* y, const int* N, int M, int K, int out_dtype, void* ws,
              size_t wsb, void* stream)
{
    if (!x || !W || !y || !N || (bits && (!scales || !biases))) return AQG_ERR_INVALID_ARG;
    if (P < 1 || P > aqg::kMaxSegments) return AQG_ERR_UNSUPPORTED;
    int64_t total = 0;
    bool aligned16 = true;
    for (int p = 0; p < P; ++p) {
        if (N[p] <= 0) return AQG_ERR_INVALID_ARG;
        if (p + 1 < P && N[p] % 16 != 0) aligned16 = false;
        total += N[p];
    }
    if (total > 0x7FFFFFFF) return AQG_ERR_UNSUPPORTED;
    // every projection is a valid call on its own (same checks, in order)
    for (int p = 0; p < P; ++p) {
        int st = check_common(x, y[p], M, N[p], K, out_dtype);
        if (st != AQG_OK) return st;
        if (!W[p] || (bits && (!scales[p] || !biases[p]))) return AQG_ERR_INVALID_ARG;
        if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return AQG_ERR_UNSUPPORTED;
        if (!aligned(W[p], 16) || (bits && (!aligned(scales[p], 4) || !aligned(biases[p], 4))))
            return AQG_ERR_ALIGNMENT;
    }
    if (wsb < aqg_workspace_bytes(bits, M, (int)total, K)) return AQG_ERR_INVALID_ARG;
    (void)ws;
    // no output overlaps an input or another output
    const size_t xbytes = (size_t)M * K * 2;
    for (int p = 0; p < P; ++p) {
        const size_t yb = out_bytes(M, N[p], out_dtype);
        if (overlap(y[p], yb, x, xbytes)) return AQG_ERR_INVALID_ARG;
        for (int q = 0; q < P; ++q) {
            const size_t wb = bits ? (size_t)N[q] * K / 8 * bits : (size_t)N[q] * K * 2;
            const size_t gb = (size_t)N[q] * (K / 64) * 2;
            if (overlap(y[p], yb, W[q], wb)) return AQG_ERR_INVALID_ARG;
            if (bits && (overlap(y[p], yb, scales[q], gb) || overlap(y[p], yb, biases[q], gb)))
                return AQG_ERR_INVALID_ARG;
            if (q != p && overlap(y[p], yb, y[q], out_bytes(M, N[q], out_dtype))) return AQG_ERR_INVALID_ARG;
        }
    }
    int st = check_device();
    if (st != AQG_OK) return st;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto base_args = [&](const aqg::LaunchCfg& cfg, int n) {
        aqg::ProjArgs a{};
        a.x = static_cast<const uint16_t*>(x);
        a.M = M;
        a.N = n;
        a.K = K;
        a.KT = cfg.KT;
        a.lpr_log2 = cfg.lpr_log2;
        a.ksplit_log2 = cfg.ksplit_log2;
        a.tpw = cfg.tpw;
        a.out_f32 = out_dtype == AQG_OUT_F32;
        return a;
    };
    const aqg::LaunchCfg cfg = aqg::choose_config(bits, false, M, (int)total, K);
    if (aligned16 && multi_fused(cfg)) {
        aqg::ProjArgs a = base_args(cfg, (int)total);
        a.nseg = P;
        int64_t row0 = 0;
        for (int p = 0; p < P; ++p) {
            a.seg_row0[p] = row0;
            a.seg_w[p] = W[p];
            a.seg_scales[p] = bits ? static_cast<const uint16_t*>(scales[p]) : nullptr;
            a.seg_biases[p] = bits ? static_cast<const uint16_t*>(biases[p]) : nullptr;
            a.seg_y[p] = y[p];
            row0 += N[p];
        }
        a.seg_row0[P] = row0;
        a.w0 = W[0];
        a.scales = a.seg_scales[0];
        a.biases = a.seg_biases[0];
        a.y = y[0];
        return finish(aqg::launch_proj(bits, false, a, cfg, s));
    }
    // otherwise one launch per projection, each on its own kernel
    for (int p = 0; p < P; ++p) {
        const aqg::LaunchCfg c = aqg::choose_config(bits, false, M, N[p], K);
        aqg::ProjArgs a = base_args(c, N[p]);
        a.w0 = W[p];
        a.scales = bits ? static_cast<const uint16_t*>(scales[p]) : nullptr;
        a.biases = bits ? static_cast<const uint16_t*>(biases[p]) : nullptr;
        a.y = y[p];
        const int e = finish(aqg::launch_proj(bits, false, a, c, s));
        if (e != AQG_OK) return e;
    }
    return AQG_OK;
}

// ---------------------------------------------------------- row argmax

constexpr int kArgmaxChunk = 8192;        // columns per partial when the GEMV writes y first
constexpr int kArgmaxRowsCap = 32;        // partial rows in the workspace (M <= 32)
constexpr int kArgmaxProducersPerCu = 32; // wavefront slots per CU: no kernel launches more

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// How a row-argmax call runs and the workspace it needs: with a fused
// epilogue the kernel writes (value, index) partials per producer; otherwise
// the GEMV writes fp32 y into the workspace and a row reduction makes the
// partials (one per column chunk).
struct ArgmaxPlan {
    bool fused;
    size_t ybytes;     // fp32 y in front of the partials (0 when fused)
    int64_t slots;     // partials per row
    size_t bytes;      // total workspace
};

ArgmaxPlan argmax_plan(int bits, int M, int N, int K)
{
    ArgmaxPlan p{};
    const aqg::LaunchCfg cfg = aqg::choose_config(bits, false, M, N, K);
    p.fused = aqg::argmax_fused(cfg);
    if (p.fused) {
        int cus = 256;
        if (aqg::detail::device_cus(cus) != hipSuccess) {
            (void)hipGetLastError();
            cus = 256;
        }
        p.ybytes = 0;
        p.slots = (int64_t)kArgmaxProducersPerCu * cus;
    } else {
        p.ybytes = round_up((size_t)M * N * 4, 256);
        p.slots = ((int64_t)N + kArgmaxChunk - 1) / kArgmaxChunk;
    }
    p.bytes = p.ybytes + (size_t)kArgmaxRowsCap * p.slots * 8;
    return p;
}

int run_argmax(int bits, const void* x, const void* w0, const void* scales, const void* biases, float* val,
               int32_t* idx, int M, int N, int K, void* ws, size_t wsb, void* stream)
{
    if (!x || !w0 || !val || !idx || (bits && (!scales || !biases))) return AQG_ERR_INVALID_ARG;
    if (M <= 0 || N <= 0 || K <= 0) return AQG_ERR_INVALID_ARG;
    if (M > 32) return AQG_ERR_UNSUPPORTED;
    if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return AQG_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w0, 16) || !aligned(val, 4) || !aligned(idx, 4)) return AQG_ERR_ALIGNMENT;
    if (bits && (!aligned(scales, 4) || !aligned(biases, 4))) return AQG_ERR_ALIGNMENT;
    const ArgmaxPlan plan = argmax_plan(bits, M, N, K);
    if (!ws || wsb < plan.bytes) return AQG_ERR_INVALID_ARG;
    if (!aligned(ws, 16)) return AQG_ERR_ALIGNMENT;
    const size_t xbytes = (size_t)M * K * 2;
    const size_t wbytes = bits ? (size_t)N * K / 8 * bits : (size_t)N * K * 2;
    const size_t gbytes = (size_t)N * (K / 64) * 2;
    const size_t ob = (size_t)M * 4;
    const void* ins[4] = {x, w0, bits ? scales : nullptr, bits ? biases : nullptr};
    const size_t insz[4] = {xbytes, wbytes, gbytes, gbytes};
    const void* outs[3] = {val, idx, ws};
    const size_t outsz[3] = {ob, ob, plan.bytes};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], outsz[o], ins[i], insz[i])) return AQG_ERR_INVALID_ARG;
        for (int p = o + 1; p < 3; ++p)
            if (overlap(outs[o], outsz[o], outs[p], outsz[p])) return AQG_ERR_INVALID_ARG;
    }
    int st = check_device();
    if (st != AQG_OK) return st;

    const aqg::LaunchCfg cfg = aqg::choose_config(bits, false, M, N, K);
    aqg::ProjArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w0 = w0;
    a.scales = static_cast<const uint16_t*>(scales);
    a.biases = static_cast<const uint16_t*>(biases);
    a.M = M;
    a.N = N;
    a.K = K;
    a.KT = cfg.KT;
    a.lpr_log2 = cfg.lpr_log2;
    a.ksplit_log2 = cfg.ksplit_log2;
    a.tpw = cfg.tpw;
    a.out_f32 = 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char* part = static_cast<char*>(ws) + plan.ybytes;
    hipError_t e;
    if (plan.fused) {
        int64_t producers = 0;
        a.y = nullptr;
        a.amx = part;
        a.amx_slots = plan.slots;
        a.amx_producers = &producers;
        e = aqg::launch_proj(bits, false, a, cfg, s);
        if (e == hipSuccess) e = aqg::launch_argmax_final(part, plan.slots, producers, M, val, idx, s);
    } else {
        a.y = ws;
        e = aqg::launch_proj(bits, false, a, cfg, s);
        if (e == hipSuccess) e = aqg::launch_argmax_rows(static_cast<const float*>(ws), M, N, kArgmaxChunk, part,
                                                         plan.slots, s);
        if (e == hipSuccess) e = aqg::launch_argmax_final(part, plan.slots, plan.slots, M, val, idx, s);
    }
    return finish(e);
}

// ------------------------------------------- argmax without allocation

// Scratch of the allocation-free row argmax: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes its
// name to a kernel (on the host it is only a stand-in for the symbol): the
// first call on a device looks up that device's address with
// hipGetSymbolAddress and every later call on it uses that pointer.
constexpr size_t kScratchBytes = AQG_ARGMAX_NOALLOC_MAX_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];      // per device: the array's device address (null until looked up)

int scratch_for_current_device(void** p)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return AQG_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return AQG_ERR_DEVICE;
        }
        g_scratch[dev] = ptr;
    }
    *p = g_scratch[dev];
    return AQG_OK;
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
        case AQG_ERR_UNSUPPORTED: return "AQG_ERR_UNSUPPORTED: M > 32 (M > AQG_GEMM_MAX_M for the prompt "
                                         "GEMMs), K not a multiple of 8 (dense) or 64 (affine), or bits "
                                         "outside 2..8";
        case AQG_ERR_ALIGNMENT: return "AQG_ERR_ALIGNMENT: x and W/Wq must be 16-byte aligned, scales and "
                                       "biases 4-byte aligned, other arrays aligned to their element size";
        case AQG_ERR_LAUNCH: return "AQG_ERR_LAUNCH: the kernel launch failed";
        case AQG_ERR_DEVICE: return "AQG_ERR_DEVICE: no current HIP device, or it is not gfx950";
        default: return "unknown aqg status";
    }
}

size_t aqg_workspace_bytes(int kind, int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    if (kind >= AQG_KIND_GEMM_AFFINE + 2 && kind <= AQG_KIND_GEMM_AFFINE + 8)
        return M > AQG_GEMM_MAX_M || K % 64 != 0 ? 0 : aqg::gemm_workspace_bytes(kind - AQG_KIND_GEMM_AFFINE, M, N, K);
    if (M > 32) return 0;
    if (kind == AQG_KIND_ARGMAX_DENSE || (kind >= AQG_KIND_ARGMAX_DENSE + 2 && kind <= AQG_KIND_ARGMAX_DENSE + 8))
        return argmax_plan(kind - AQG_KIND_ARGMAX_DENSE, M, N, K).bytes;
    return 0;  // the GEMVs and SwiGLUs keep their partial sums in registers and LDS
}

int aqg_gemv_argmax_noalloc(int bits, const void* x, const void* W, const void* scales, const void* biases,
                            float* max_val, int32_t* max_idx, int M, int N, int K, void* stream)
{
    if (!(bits == 0 || (bits >= 2 && bits <= 8))) return AQG_ERR_UNSUPPORTED;
    if (M <= 0 || N <= 0 || K <= 0) return AQG_ERR_INVALID_ARG;
    if (M > 32) return AQG_ERR_UNSUPPORTED;
    if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return AQG_ERR_UNSUPPORTED;
    if (argmax_plan(bits, M, N, K).bytes > kScratchBytes) return AQG_ERR_UNSUPPORTED;
    int st = check_device();
    if (st != AQG_OK) return st;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != AQG_OK) return st;
    return run_argmax(bits, x, W, scales, biases, max_val, max_idx, M, N, K, ws, kScratchBytes, stream);
}

int aqg_gemv_bf16_multi(const void* x, int P, const void* const* W, void* const* y, const int* N, int M, int K,
                        int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return run_multi(0, x, P, W, nullptr, nullptr, y, N, M, K, out_dtype, workspace, workspace_bytes, stream);
}

#define AQG_AFFINE_MULTI_ENTRY(B)                                                                            \
    int aqg_gemv_affine_q##B##_multi(const void* x, int P, const uint32_t* const* Wq,                        \
                                     const void* const* scales, const void* const* biases, void* const* y,  \
                                     const int* N, int M, int K, int out_dtype, void* workspace,            \
                                     size_t workspace_bytes, void* stream)                                  \
    {                                                                                                        \
        return run_multi(B, x, P, reinterpret_cast<const void* const*>(Wq), scales, biases, y, N, M, K,      \
                         out_dtype, workspace, workspace_bytes, stream);                                     \
    }
AQG_AFFINE_MULTI_ENTRY(2)
AQG_AFFINE_MULTI_ENTRY(3)
AQG_AFFINE_MULTI_ENTRY(4)
AQG_AFFINE_MULTI_ENTRY(5)
AQG_AFFINE_MULTI_ENTRY(6)
AQG_AFFINE_MULTI_ENTRY(7)
AQG_AFFINE_MULTI_ENTRY(8)
#undef AQG_AFFINE_MULTI_ENTRY

int aqg_gemv_bf16_argmax(const void* x, const void* W, float* max_val, int32_t* max_idx, int M, int N, int K,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    return run_argmax(0, x, W, nullptr, nullptr, max_val, max_idx, M, N, K, workspace, workspace_bytes, stream);
}

#define AQG_AFFINE_ARGMAX_ENTRY(B)                                                                          \
    int aqg_gemv_affine_q##B##_argmax(const void* x, const uint32_t* Wq, const void* scales,               \
                                      const void* biases, float* max_val, int32_t* max_idx, int M, int N,  \
                                      int K, void* workspace, size_t workspace_bytes, void* stream)        \
    {                                                                                                       \
        return run_argmax(B, x, Wq, scales, biases, max_val, max_idx, M, N, K, workspace, workspace_bytes,  \
                          stream);                                                                          \
    }
AQG_AFFINE_ARGMAX_ENTRY(2)
AQG_AFFINE_ARGMAX_ENTRY(3)
AQG_AFFINE_ARGMAX_ENTRY(4)
AQG_AFFINE_ARGMAX_ENTRY(5)
AQG_AFFINE_ARGMAX_ENTRY(6)
AQG_AFFINE_ARGMAX_ENTRY(7)
AQG_AFFINE_ARGMAX_ENTRY(8)
#undef AQG_AFFINE_ARGMAX_ENTRY

int aqg_gemv_bf16(const void* x, const void* W, void* y, int M, int N, int K, int out_dtype,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    return run_projection(0, false, x, W, nullptr, nullptr, nullptr, nullptr, nullptr, y, M, N, K, out_dtype,
                          workspace, workspace_bytes, stream);
}

int aqg_swiglu_bf16(const void* x, const void* Wg, const void* Wu, void* out, int M, int N, int K,
                    int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return run_projection(0, true, x, Wg, Wu, nullptr, nullptr, nullptr, nullptr, out, M, N, K, out_dtype,
                          workspace, workspace_bytes, stream);
}

#define AQG_SWIGLU_AFFINE_ENTRY(B)                                                                          \
    int aqg_swiglu_affine_q##B(const void* x, const uint32_t* Wgq, const void* gate_scales,                 \
                               const void* gate_biases, const uint32_t* Wuq, const void* up_scales,        \
                               const void* up_biases, void* out, int M, int N, int K, int out_dtype,       \
                               void* workspace, size_t workspace_bytes, void* stream)                      \
    {                                                                                                       \
        return run_projection(B, true, x, Wgq, Wuq, gate_scales, gate_biases, up_scales, up_biases, out, M, \
                              N, K, out_dtype, workspace, workspace_bytes, stream);                         \
    }
AQG_SWIGLU_AFFINE_ENTRY(2)
AQG_SWIGLU_AFFINE_ENTRY(3)
AQG_SWIGLU_AFFINE_ENTRY(4)
AQG_SWIGLU_AFFINE_ENTRY(5)
AQG_SWIGLU_AFFINE_ENTRY(6)
AQG_SWIGLU_AFFINE_ENTRY(7)
AQG_SWIGLU_AFFINE_ENTRY(8)
#undef AQG_SWIGLU_AFFINE_ENTRY

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

#define AQG_GEMM_ENTRY(B)                                                                            \
    int aqg_gemm_affine_q##B(const void* x, const uint32_t* Wq, const void* scales, const void* biases, \
                             void* y, int M, int N, int K, int out_dtype, void* workspace,          \
                             size_t workspace_bytes, void* stream)                                  \
    {                                                                                                \
        return run_gemm(B, x, Wq, scales, biases, y, M, N, K, out_dtype, workspace, workspace_bytes, \
                        stream);                                                                     \
    }
AQG_GEMM_ENTRY(2)
AQG_GEMM_ENTRY(3)
AQG_GEMM_ENTRY(4)
AQG_GEMM_ENTRY(5)
AQG_GEMM_ENTRY(6)
AQG_GEMM_ENTRY(7)
AQG_GEMM_ENTRY(8)
#undef AQG_GEMM_ENTRY

int aqg_dispatch_path(int kind, int M, int N, int K, int* columns)
{
    if (M <= 0 || N <= 0 || K <= 0) return -AQG_ERR_INVALID_ARG;
    if (kind >= AQG_KIND_GEMM_AFFINE + 2 && kind <= AQG_KIND_GEMM_AFFINE + 8) {
        if (M > AQG_GEMM_MAX_M || K % 64 != 0) return -AQG_ERR_UNSUPPORTED;
        if (columns) *columns = aqg::kGemmTileM;
        return aqg::PATH_AFFINE_GEMM;
    }
    const bool swiglu_affine = kind >= AQG_KIND_SWIGLU_AFFINE + 2 && kind <= AQG_KIND_SWIGLU_AFFINE + 8;
    const bool swiglu = kind == AQG_KIND_SWIGLU || swiglu_affine;
    const int bits = swiglu_affine ? kind - AQG_KIND_SWIGLU_AFFINE : (swiglu ? 0 : kind);
    if (!(kind == AQG_KIND_DENSE || swiglu || (kind >= 2 && kind <= 8))) return -AQG_ERR_INVALID_ARG;
    if (M > 32) return -AQG_ERR_UNSUPPORTED;
    if (bits == 0 ? (K % 8 != 0) : (K % 64 != 0)) return -AQG_ERR_UNSUPPORTED;
    // no device check: without a device the geometry assumes 256 CUs
    const aqg::LaunchCfg cfg = aqg::choose_config(bits, swiglu, M, N, K);
    if (columns) *columns = cfg.MT;
    return cfg.path;
}

const char* aqg_path_name(int path)
{
    switch (path) {
        case aqg::PATH_VALU: return "valu";
        case aqg::PATH_MFMA: return "mfma";
        case aqg::PATH_STREAM: return "stream";
        case aqg::PATH_PIECE: return "piece";
        case aqg::PATH_MFMA_STREAM: return "mfma_stream";
        case aqg::PATH_MFMA_SPLIT: return "mfma_split";
        case aqg::PATH_AFFINE_MFMA: return "affine_mfma";
        case aqg::PATH_MFMA_TILE: return "mfma_tile";
        case aqg::PATH_AFFINE_TILE: return "affine_tile";
        case aqg::PATH_AFFINE_SPLIT: return "affine_split";
        case aqg::PATH_AFFINE_BURST: return "affine_burst";
        case aqg::PATH_AFFINE_GEMM: return "affine_gemm";
        default: return "unknown";
    }
}

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
