/*
 * oracle.c -- plain, slow, double-precision CPU reference for the small-M
 * decode projections: dense bf16 GEMV, affine group-quantized GEMV (2..8-bit
 * codes, groups of 64 along K, bf16 scale and bias per group) and the fused
 * up/gate SwiGLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It exists so that the GPU kernels can be checked
 * against the plain definition of what they compute.  It shares no code, no
 * header and no table with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *  - TensorFold PR #849, "qwen3_5 cuda: mixed-width MLX checkpoints, 2 to 8
 *    bits in groups of 64": the weight format -- MLX affine mode, each module
 *    at a width from 2 to 8 bits, groups of 64, every code keeping its value,
 *    scale and bias (the "What this changes" body and the widths comment).
 *  - AstrAI decode_linear_benchmark.md, commit message: the fused BF16 up/gate
 *    SwiGLU primitive, silu(x Wg^T) * (x Wu^T), against the unfused chain.
 *  - nvfp4-megamoe-kernel commit log, "Router: full kernel stack", Step 2
 *    (topk_select): on equal scores the lower index wins.
 *  - same commit, closing "Test strategy" paragraph: the oracle is the math.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - Affine form: w = scale * q + bias (MLX affine; no zero-point).
 *  - Bit layout: one LSB-first bit stream per row; code k of a row occupies
 *    stream bits [b*k, b*k + b); stream bit j is bit (j & 31) of uint32 word
 *    (j >> 5) of that row.  A row holds K*b/32 words.
 *  - scales and biases: two bf16 arrays of shape [N, K/64], row-major.
 *  - All arithmetic below is IEEE double, sums in ascending k.
 *
 * Parallelism: OpenMP over output rows n only, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 */

/* bf16 bit pattern -> double.  Exact: a bf16 is the upper half of a float. */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* float -> bf16, round to nearest, ties to even.  NaN maps to the quiet NaN
 * 0x7FC0 with the input's sign. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Vector form of the two conversions above (for the tests' exhaustive sweep
 * and for reference rounding of GPU fp32 outputs). */
void oracle_f32_to_bf16_vec(const float *in, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_bf16_to_double_vec(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_double(in[i]);
}

/* ------------------------------------------------------- pack / unpack */

static int bits_ok(int bits) { return bits >= 2 && bits <= 8; }

/* codes[N][K] (uint8, each < 2^bits) -> words[N][K*bits/32].
 * Bit i of code k is stream bit bits*k + i.  Returns 0 on success. */
int oracle_pack(int bits, const uint8_t *codes, uint32_t *words, int64_t N, int64_t K)
{
    if (!bits_ok(bits) || (K * bits) % 32 != 0)
        return 1;
    int64_t wpr = K * bits / 32;
    memset(words, 0, (size_t)(N * wpr) * sizeof(uint32_t));
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = words + n * wpr;
        for (int64_t k = 0; k < K; ++k) {
            unsigned c = codes[n * K + k];
            for (int i = 0; i < bits; ++i) {
                if ((c >> i) & 1u) {
                    int64_t j = (int64_t)bits * k + i;
                    row[j >> 5] |= 1u << (j & 31);
                }
            }
        }
    }
    return 0;
}

/* One code, written independently of oracle_pack: take the 32-bit word that
 * holds the code's first bit, shift it down, and if the code runs past that
 * word, bring its high bits in from the next word. */
static unsigned unpack_one(const uint32_t *row, int bits, int64_t k)
{
    int64_t off = (int64_t)bits * k;
    int64_t w = off >> 5;
    int s = (int)(off & 31);
    uint32_t v = row[w] >> s;
    if (s + bits > 32)
        v |= row[w + 1] << (32 - s);
    return v & ((1u << bits) - 1u);
}

int oracle_unpack(int bits, const uint32_t *words, uint8_t *codes, int64_t N, int64_t K)
{
    if (!bits_ok(bits) || (K * bits) % 32 != 0)
        return 1;
    int64_t wpr = K * bits / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)unpack_one(words + n * wpr, bits, k);
    return 0;
}

/* --------------------------------------------------------------- GEMVs */

/* y[m][n] = sum_k W[n][k] * x[m][k];  A[m][n] = sum_k |W[n][k] * x[m][k]|.
 * x: bf16[M][K]; W: bf16[N][K]; y, A: double[M][N] (A may be NULL). */
void oracle_gemv_bf16(const uint16_t *x, const uint16_t *W, double *y, double *A,
                      int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = oracle_bf16_to_double(W[n * K + k]);
                double xv = oracle_bf16_to_double(x[m * K + k]);
                double p = w * xv;
                acc += p;
                aacc += fabs(p);
            }
            y[m * N + n] = acc;
            if (A)
                A[m * N + n] = aacc;
        }
    }
}

/* Affine dequantization of one weight: w = scale * q + bias, in double.
 * scale * q is exact (8-bit significand times an integer below 256); the sum
 * with the bias is exact whenever the two exponents are within ~37 of each
 * other, which holds for every input the tests draw. */
static double dequant(int bits, const uint32_t *row_words, const uint16_t *row_scales,
                      const uint16_t *row_biases, int64_t k)
{
    unsigned q = unpack_one(row_words, bits, k);
    double s = oracle_bf16_to_double(row_scales[k / 64]);
    double b = oracle_bf16_to_double(row_biases[k / 64]);
    return s * (double)q + b;
}

/* Affine GEMV.  Wq: uint32[N][K*bits/32]; scales, biases: bf16[N][K/64].
 * Returns 0 on success, 1 on a shape the format does not allow. */
int oracle_gemv_affine(int bits, const uint16_t *x, const uint32_t *Wq,
                       const uint16_t *scales, const uint16_t *biases,
                       double *y, double *A, int64_t M, int64_t N, int64_t K)
{
    if (!bits_ok(bits) || K % 64 != 0)
        return 1;
    int64_t wpr = K * bits / 32, gpr = K / 64;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *rw = Wq + n * wpr;
        const uint16_t *rs = scales + n * gpr;
        const uint16_t *rb = biases + n * gpr;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = dequant(bits, rw, rs, rb, k);
                double p = w * oracle_bf16_to_double(x[m * K + k]);
                acc += p;
                aacc += fabs(p);
            }
            y[m * N + n] = acc;
            if (A)
                A[m * N + n] = aacc;
        }
    }
    return 0;
}

/* Unfused SwiGLU chain in double, no intermediate rounding:
 *   g = x Wg^T, u = x Wu^T, out = g / (1 + exp(-g)) * u.
 * g, u, Ag, Au: double[M][N] (any may be NULL except out). */
void oracle_swiglu_bf16(const uint16_t *x, const uint16_t *Wg, const uint16_t *Wu,
                        double *out, double *g, double *u, double *Ag, double *Au,
                        int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double ga = 0.0, ua = 0.0, gaa = 0.0, uaa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = oracle_bf16_to_double(x[m * K + k]);
                double pg = oracle_bf16_to_double(Wg[n * K + k]) * xv;
                double pu = oracle_bf16_to_double(Wu[n * K + k]) * xv;
                ga += pg;
                ua += pu;
                gaa += fabs(pg);
                uaa += fabs(pu);
            }
            double silu = ga / (1.0 + exp(-ga));
            int64_t i = m * N + n;
            out[i] = silu * ua;
            if (g) g[i] = ga;
            if (u) u[i] = ua;
            if (Ag) Ag[i] = gaa;
            if (Au) Au[i] = uaa;
        }
    }
}

/* Unfused SwiGLU chain over two affine b-bit matrices (the gate and up
 * projections of an MLX affine checkpoint's MLP), in double, no intermediate
 * rounding:
 *   g[m][n] = sum_k x[m][k] * (sg[n][k/64] * qg[n][k] + bg[n][k/64]),
 *   u[m][n] = the same with the up matrix,
 *   out = g / (1 + exp(-g)) * u.
 * Each matrix has its own codes, scales and biases in the layout of
 * oracle_gemv_affine; both share the width.  Ag, Au = sum_k |w x|.  g, u,
 * Ag, Au may be NULL.  Returns 0 on success, 1 on a shape the format does
 * not allow.  (AstrAI decode_linear_benchmark.md, commit message: the fused
 * up/gate SwiGLU against the unfused chain; TensorFold PR #849: the affine
 * format of the MLP modules.) */
int oracle_swiglu_affine(int bits, const uint16_t *x,
                         const uint32_t *Wgq, const uint16_t *sg, const uint16_t *bg,
                         const uint32_t *Wuq, const uint16_t *su, const uint16_t *bu,
                         double *out, double *g, double *u, double *Ag, double *Au,
                         int64_t M, int64_t N, int64_t K)
{
    if (!bits_ok(bits) || K % 64 != 0)
        return 1;
    int64_t wpr = K * bits / 32, gpr = K / 64;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double ga = 0.0, ua = 0.0, gaa = 0.0, uaa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = oracle_bf16_to_double(x[m * K + k]);
                double pg = dequant(bits, Wgq + n * wpr, sg + n * gpr, bg + n * gpr, k) * xv;
                double pu = dequant(bits, Wuq + n * wpr, su + n * gpr, bu + n * gpr, k) * xv;
                ga += pg;
                ua += pu;
                gaa += fabs(pg);
                uaa += fabs(pu);
            }
            double silu = ga / (1.0 + exp(-ga));
            int64_t i = m * N + n;
            out[i] = silu * ua;
            if (g) g[i] = ga;
            if (u) u[i] = ua;
            if (Ag) Ag[i] = gaa;
            if (Au) Au[i] = uaa;
        }
    }
    return 0;
}

/* Row-wise argmax over y[M][N]; the lowest index wins on equal values. */
void oracle_argmax(const double *y, int64_t *idx, int64_t M, int64_t N)
{
    for (int64_t m = 0; m < M; ++m) {
        int64_t best = 0;
        for (int64_t n = 1; n < N; ++n)
            if (y[m * N + n] > y[m * N + best])
                best = n;
        idx[m] = best;
    }
}

void oracle_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
