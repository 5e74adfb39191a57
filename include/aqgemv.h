/*
 * aqgemv.h -- C ABI of libaqgemv.so: small-M decode projections on AMD
 * Instinct MI355X (gfx950).
 *
 *   y[M,N] = x[M,K] . W^T          W dense bf16            (aqg_gemv_bf16)
 *   y[M,N] = x[M,K] . W^T          W affine b-bit, b=2..8  (aqg_gemv_affine_q2 .. _q8)
 *   out[M,N] = silu(x.Wg^T) * (x.Wu^T)                     (aqg_swiglu_bf16)
 *
 * for M = 1..32 rows of activations (single-stream decode, or a window of up
 * to 32 rows).
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
 *  - M in [1, 32]; N, K >= 1.  Dense: K % 8 == 0.  Affine: K % 64 == 0.
 *    x and W/Wq must be 16-byte aligned; scales and biases 4-byte aligned
 *    (read in 4- to 16-byte pieces); y and codes naturally aligned for their
 *    element type.  y must not overlap any input.
 *  - out_dtype AQG_OUT_F32 writes the fp32 sums; AQG_OUT_BF16 writes exactly
 *    the round-to-nearest-even bf16 of the values the same call would write
 *    with AQG_OUT_F32 (kernels are deterministic).
 *  - workspace: scratch for split-K variants.  aqg_workspace_bytes() gives the
 *    size a call needs; NULL / 0 is valid when that size is 0, otherwise a
 *    smaller workspace is AQG_ERR_INVALID_ARG.
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
#define AQG_KIND_DENSE 0   /* 2..8 = affine of that width */
#define AQG_KIND_SWIGLU 9

/* Returns AQG_ABI_VERSION. */
int aqg_abi_version(void);

/* Static description of a status code (never NULL). */
const char* aqg_status_string(int status);

/* Workspace bytes a call of the given kind and shape needs (0 = none). */
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
 * Unpack codes: codes[n][k] = q[n,k] as uint8, through the same device code
 * path the affine GEMVs use to read their weights.  Wq: uint32[N][K*b/32];
 * codes: uint8[N][K].  K % 64 == 0.  A test hook for bit-exact checks.
 */
int aqg_unpack_codes(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AQGEMV_H */
