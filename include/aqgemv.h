/*
 * aqgemv.h -- C ABI of libaqgemv.so: small-M decode projections on AMD
 * Instinct MI355X (gfx950).
 *
 *   y[M,N] = x[M,K] . W^T          W dense bf16            (aqg_gemv_bf16)
 *   y[M,N] = x[M,K] . W^T          W affine b-bit, b=2..8  (aqg_gemv_affine_q2 .. _q8)
 *   out[M,N] = silu(x.Wg^T) * (x.Wu^T)   Wg, Wu dense      (aqg_swiglu_bf16)
 *                                        Wg, Wu affine     (aqg_swiglu_affine_q2 .. _q8)
 *   argmax over n of y[m,n], without writing y             (aqg_gemv_*_argmax)
 *
 * for M = 1..32 rows of activations (single-stream decode, or a window of up
 * to 32 rows), and the affine product for any M (prompt chunks):
 *   y[M,N] = x[M,K] . W^T          W affine b-bit, M >= 1  (aqg_gemm_affine_q2 .. _q8)
 *
 * Sources (web pages, cited by title and section):
 *  - AstrAI decode_linear_benchmark.md -- the commit message: a BF16 GEMV for
 *    decode projections and a fused BF16 up/gate SwiGLU primitive; the page
 *    body: q/k/v/out, MLP up/gate/down and LM-head shapes at M = 1..32.
 *  - TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2 to 8
 *    bits in groups of 64" -- the affine weight format: MLX affine mode, widths
 *    2 to 8 bits, groups of 64, each code keeping its value, scale and bias;
 *    other group sizes and non-affine modes are refused.
 *
 * Affine format (the pages name it but give no formula or bit layout; these
 * are the plainest readings):
 *  - w[n,k] = scale[n, k/64] * q[n,k] + bias[n, k/64], q in [0, 2^b - 1].
 *  - Wq: uint32[N][K*b/32].  Row n is one LSB-first bit stream: code k sits
 *    at stream bits [b*k, b*k + b), and stream bit j is bit (j & 31) of word
 *    (j >> 5) of the row.  For b = 4 this is 8 codes per uint32,
 *    little-endian along K.  A group of 64 codes is exactly 2*b words.
 *  - scales, biases: two bf16 arrays [N][K/64], row-major.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; all arrays
 *    are row-major and contiguous.  bf16 is the 16-bit brain-float pattern.
 *  - The library never allocates, frees or synchronizes.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the legacy default stream) and the call
 *    returns once it is enqueued.  Device faults surface at the caller's next
 *    synchronization.
 *  - Validation happens on the host before any HIP call.  On any status other
 *    than AQG_OK nothing has been enqueued and the outputs are untouched.
 *  - M in [1, 32] (the prompt GEMMs: [1, AQG_GEMM_MAX_M]); N, K >= 1.
 *    Dense: K % 8 == 0.  Affine: K % 64 == 0.
 *    x and W/Wq must be 16-byte aligned; scales and biases 4-byte aligned
 *    (read in 4- to 16-byte pieces); y and codes naturally aligned for their
 *    element type.  y must not overlap any input.
 *  - out_dtype AQG_OUT_F32 writes the fp32 sums; AQG_OUT_BF16 writes exactly
 *    the round-to-nearest-even bf16 of the values the same call would write
 *    with AQG_OUT_F32 (kernels are deterministic).
 *  - workspace: scratch of the calls that need one (the row argmax, the
 *    prompt GEMMs).
 *    aqg_workspace_bytes() gives the size a call needs; NULL / 0 is valid
 *    when that size is 0, otherwise a smaller workspace is
 *    AQG_ERR_INVALID_ARG (the prompt GEMMs also accept less, down to what
 *    their operands need: see there).
 *  - Accumulation is fp32; the result of each (m, n) does not depend on M
 *    within one code path (rows are independent).
 *  - Thread safety: stateless apart from a per-device architecture check that
 *    is cached on first use; calls may be made from several threads.
 */
#ifndef AQGEMV_H
#define AQGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AQG_ABI_VERSION 1

/* Status codes returned by every entry point. */
typedef enum {
    AQG_OK = 0,
    AQG_ERR_INVALID_ARG = 1,  /* null pointer, size <= 0, bad out_dtype, short workspace, overlap */
    AQG_ERR_UNSUPPORTED = 2,  /* M > 32, K not a multiple of 8 (dense) / 64 (affine), bits not 2..8 */
    AQG_ERR_ALIGNMENT = 3,    /* a pointer is not aligned as required above */
    AQG_ERR_LAUNCH = 4,       /* the HIP launch reported an error */
    AQG_ERR_DEVICE = 5        /* no current HIP device, or it is not gfx950 */
} aqg_status;

typedef enum { AQG_OUT_BF16 = 0, AQG_OUT_F32 = 1 } aqg_out_dtype;

/* Kinds for aqg_workspace_bytes(). */
#define AQG_KIND_DENSE 0           /* 2..8 = affine GEMV of that width */
#define AQG_KIND_SWIGLU 9
#define AQG_KIND_SWIGLU_AFFINE 16  /* + b (2..8) = affine SwiGLU of width b */
#define AQG_KIND_ARGMAX_DENSE 32   /* + b (2..8) = affine row argmax of width b */
#define AQG_KIND_GEMM_AFFINE 48    /* + b (2..8) = affine prompt GEMM of width b (any M) */

/* Returns AQG_ABI_VERSION. */
int aqg_abi_version(void);

/* Static description of a status code (never NULL). */
const char* aqg_status_string(int status);

/* Workspace bytes a call of the given kind and shape needs (0 = none).
 * Asked of the library before a call rather than assumed: a split-K test
 * that passed a null partials buffer wrote through it (TensorFold PR #849,
 * the split-K fix in the PR body).  The library checks the size it is given
 * against this value and refuses a shorter one. */
size_t aqg_workspace_bytes(int kind, int M, int N, int K);

/*
 * Dense bf16 GEMV: y[m,n] = sum_k x[m,k] * W[n,k], fp32 accumulation.
 *   x: bf16[M][K]; W: bf16[N][K]; y: bf16 or f32 [M][N] per out_dtype.
 * AstrAI decode_linear_benchmark.md, commit message (BF16 decode GEMV).
 */
int aqg_gemv_bf16(const void* x, const void* W, void* y, int M, int N, int K,
                  int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Affine group-quantized GEMV of width b (one symbol per b = 2..8):
 *   y[m,n] = sum_k x[m,k] * (scale[n,k/64] * q[n,k] + bias[n,k/64]),
 * fp32 accumulation; scale and bias are applied in fp32 (dequantized weights
 * are never rounded to bf16).
 *   x: bf16[M][K]; Wq: uint32[N][K*b/32] (layout above);
 *   scales, biases: bf16[N][K/64]; y: bf16 or f32 [M][N].
 * TensorFold PR #849 (format; "2 to 8 bits, in groups of 64").
 */
int aqg_gemv_affine_q2(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q3(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q4(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q5(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q6(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q7(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q8(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused up/gate SwiGLU: g = x.Wg^T, u = x.Wu^T (fp32), out = g/(1+exp(-g)) * u
 * in fp32, stored per out_dtype.  x: bf16[M][K]; Wg, Wu: bf16[N][K];
 * out: bf16 or f32 [M][N].
 * AstrAI decode_linear_benchmark.md, commit message (fused BF16 up/gate
 * SwiGLU primitive).
 */
int aqg_swiglu_bf16(const void* x, const void* Wg, const void* Wu, void* out, int M, int N, int K,
                    int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused up/gate SwiGLU over two affine b-bit matrices (one symbol per
 * b = 2..8): g = x . Wg^T and u = x . Wu^T with w = scale * q + bias per
 * group of 64 (each matrix with its own codes, scales and biases, in the
 * affine layout above), both in fp32 from the same x; out = g/(1+exp(-g)) * u
 * in fp32, stored per out_dtype.  Neither g nor u is rounded or written.
 *   x: bf16[M][K]; Wgq, Wuq: uint32[N][K*b/32]; gate_scales, gate_biases,
 *   up_scales, up_biases: bf16[N][K/64]; out: bf16 or f32 [M][N].
 * AstrAI decode_linear_benchmark.md, commit message (the fused up/gate
 * SwiGLU primitive against the unfused chain) on the affine format of
 * TensorFold PR #849 (MLX checkpoints quantize the MLP modules at the width
 * their quantization table names).
 */
int aqg_swiglu_affine_q2(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q3(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q4(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q5(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q6(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q7(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_swiglu_affine_q8(const void* x, const uint32_t* Wgq, const void* gate_scales, const void* gate_biases,
                         const uint32_t* Wuq, const void* up_scales, const void* up_biases, void* out, int M,
                         int N, int K, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several projections of the same x in one launch (e.g. the q, k and v
 * projections of an attention layer): for p < P,
 *   y_p[m, n] = sum_k x[m,k] * W_p[n,k]      (n < N[p]),
 * fp32 accumulation, within the GEMV bound.  When the launch is fused every
 * output has exactly the bits of the same row of a single call on the
 * concatenated matrix (rows of W_0, then W_1, ...): the same kernel computes
 * it.  Small decode
 * projections cost launch and first-load latency more than bandwidth; a
 * forward's launches captured once and replayed cut a 2B model's decode
 * step from 5.3 to 2.8 ms (TensorFold PR #849, the note on captured
 * forwards), and a decode step can run as one persistent dispatch for the
 * same reason (luce-megakernel HANDOFF.md, Architecture Summary).
 *   P in 1..4; W, (scales, biases), y, N: host arrays of P entries (read
 *   during the call) holding device pointers and row counts; every
 *   projection must be a valid call on its own, and no output may overlap
 *   an input or another output.
 * One kernel serves all P projections when the shape of their concatenation
 * (N = sum of N[p]) runs on a kernel that takes a projection table (the
 * 16-byte-piece dot-product kernel or a small-matrix matrix-core kernel)
 * and N[0..P-2] are multiples of 16; otherwise the projections are launched
 * one after another on the same stream.
 */
int aqg_gemv_bf16_multi(const void* x, int P, const void* const* W, void* const* y, const int* N, int M, int K,
                        int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q2_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q3_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q4_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q5_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q6_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q7_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q8_multi(const void* x, int P, const uint32_t* const* Wq, const void* const* scales,
                             const void* const* biases, void* const* y, const int* N, int M, int K,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Row argmax of a projection (the LM head of greedy decoding), without
 * writing the logits: for each row m < M,
 *   max_idx[m] = the lowest n with y[m,n] = max over n' of y[m,n'],
 *   max_val[m] = y[m, max_idx[m]],
 * where y is the fp32 result the GEMV of the same arguments writes with
 * AQG_OUT_F32 (the same kernels and arithmetic; only the epilogue differs).
 * The lower index wins on equal values (nvfp4-megamoe-kernel commit log,
 * "Router: full kernel stack", Step 2, topk_select); the draw happens on the
 * device, as the served decoder does (TensorFold PR #849, the note on the
 * MLX affine 4-bit checkpoint on the native CUDA server: sample.cu draws on
 * the device).  NaN values never win; a row of NaNs gives index INT32_MAX.
 *   max_val: float[M]; max_idx: int32[M] (device, 4-byte aligned, not
 *   overlapping any input, each other or the workspace).
 *   workspace: at least aqg_workspace_bytes(AQG_KIND_ARGMAX_DENSE (+ b), M,
 *   N, K) bytes, 16-byte aligned (required: per-producer partial maxima,
 *   and for shapes whose kernel has no argmax epilogue the fp32 y; asked of
 *   the library for the shape, since the kernel choice decides it).  Its
 *   contents on entry do not matter and are garbage afterwards.
 * Other arguments and rules as for the GEMVs above.
 */
int aqg_gemv_bf16_argmax(const void* x, const void* W, float* max_val, int32_t* max_idx, int M, int N, int K,
                         void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q2_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q3_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q4_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q5_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q6_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q7_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemv_affine_q8_argmax(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                              float* max_val, int32_t* max_idx, int M, int N, int K,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Affine prompt GEMM of width b (one symbol per b = 2..8): the same product
 * as aqg_gemv_affine_q{b},
 *   y[m,n] = sum_k x[m,k] * (scale[n,k/64] * q[n,k] + bias[n,k/64]),
 * for any number of activation rows M in [1, AQG_GEMM_MAX_M] (prompt chunks;
 * for M <= 32 the GEMVs above are the faster call).  Same arrays, layouts,
 * alignment and out_dtype rules as the GEMVs; K % 64 == 0.
 *   workspace: device memory, 16-byte aligned, not overlapping any other
 *   argument: the call writes x rearranged into matrix-core operands and the
 *   per-group sums of x there (about 2 M K bytes, always required), and,
 *   when the row tiles alone would leave a quarter of the CUs idle (N of a
 *   few thousand rows), splits each tile's groups over 2..8 workgroups whose
 *   fp32 partial products (ks M N 4 bytes) it sums in a fixed order.
 *   aqg_workspace_bytes(AQG_KIND_GEMM_AFFINE + b, M, N, K) is the size with
 *   the split on a full 256-CU gfx950; a smaller workspace that still holds
 *   the operands is accepted and runs without the split.
 * Accumulation is fp32 (per 64-code group: scale times the codes' dot
 * product, plus the bias and code-offset terms).  Row m of y depends only on
 * row m of x, W and the kernel's tiling, which is a function of ceil(M/64),
 * N, K, the CU count and whether the workspace holds the split's partial
 * products: such calls agree bit for bit on their common rows.  The result
 * is within the same bound of the exact product as the GEMVs', but not
 * bit-equal to them.
 * TensorFold PR #849 (format; the page also notes that its 8-bit modules
 * have no prompt GEMM and run prompts on the decode tiles).
 */
#define AQG_GEMM_MAX_M 65536
int aqg_gemm_affine_q2(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q3(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q4(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q5(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q6(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q7(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int aqg_gemm_affine_q8(const void* x, const uint32_t* Wq, const void* scales, const void* biases,
                       void* y, int M, int N, int K, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Row argmax that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same result as aqg_gemv_bf16_argmax
 * (bits = 0) or aqg_gemv_affine_q{bits}_argmax (bits = 2..8) with the same
 * arguments; W is the dense weight or the affine Wq, and scales and biases
 * are ignored for bits = 0.  Instead of a caller's workspace it uses a
 * static device array of AQG_ARGMAX_NOALLOC_MAX_BYTES (8 MiB) that
 * each GPU the library runs on holds until the process ends; it is looked up
 * on the first call on each device.  A shape needing more workspace than
 * that (aqg_workspace_bytes of the matching argmax kind) is
 * AQG_ERR_UNSUPPORTED; nothing is enqueued then.  The array is shared by
 * every call on a GPU: calls that may overlap on one GPU (several streams,
 * several threads) race on it and must be serialized by the caller.  Its
 * contents need no initialisation (every partial is written before it is
 * read).  No hipMalloc, hipFree or other allocating call is made.
 */
#define AQG_ARGMAX_NOALLOC_MAX_BYTES ((size_t)8 << 20)
int aqg_gemv_argmax_noalloc(int bits, const void* x, const void* W, const void* scales, const void* biases,
                            float* max_val, int32_t* max_idx, int M, int N, int K, void* stream);

/*
 * Unpack codes: codes[n][k] = q[n,k] as uint8, through the same device code
 * path the affine GEMVs use to read their weights.  Wq: uint32[N][K*b/32];
 * codes: uint8[N][K] (16-byte aligned, not overlapping Wq).  K % 64 == 0,
 * bits in 2..8.  A test hook for bit-exact checks of the bit-stream reading
 * above: every code keeps its exact value (TensorFold PR #849, "What this
 * changes" and the module-width comment).
 */
int aqg_unpack_codes(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, void* stream);

/*
 * Diagnostics (test hook; launches nothing).  The kernel family a call of
 * `kind` (AQG_KIND_DENSE, 2..8 for affine widths, AQG_KIND_SWIGLU) with
 * this shape runs on the current device (with no device: on one of 256
 * CUs, the MI355X's count), as an id >= 0 whose name
 * aqg_path_name() gives; *columns (if not NULL) receives the kernel's
 * column count (M padded).  Within one id and column count every output is
 * computed by the same chain of operations whatever M is, so tests of row
 * independence and exactness can state which kernel they cover.  Returns
 * -status (e.g. -AQG_ERR_UNSUPPORTED) for a call the library would refuse.
 */
int aqg_dispatch_path(int kind, int M, int N, int K, int* columns);
const char* aqg_path_name(int path);

/*
 * Measurement probe (launches one kernel, computes nothing): reads bytes
 * bytes from src (device, 16-byte aligned, bytes >= 16) with the weight
 * streams' access pattern (16-byte buffer loads, whole 128-byte lines per
 * instruction, eight 4-wavefront workgroups per CU) and no arithmetic.  Its
 * time over sizes gives the machine's read ceiling t0 + bytes/BW, the curve
 * the projections are reported against (the benchmark section of AstrAI
 * decode_linear_benchmark.md reports estimated effective IO bandwidth).
 * sink: a float per workgroup (8 per CU), almost never written.
 */
int aqg_stream_read(const void* src, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AQGEMV_H */
