/*
 * q4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU evaluation of the weight-only
 * 4-bit linear layer.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library; the GPU product path
 * never calls it and shares no code, header or table with it.
 *
 * What it computes (each function cites the passage it follows):
 *
 *   out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8)  (+ bias[n])
 *
 *   - Dense linear form out[m,n] = sum_k in[m,k] * weight[n,k] (+ bias[n]):
 *     page 2, "[ExecuTorch][WebGPU] Add optimized linear_fp32 op", Solution.
 *   - Signed nibble, dequant(W[n,k]) = (code - 8) * scale: page 3,
 *     "Add fp32 matmul ops (mm, bmm, linear)", stack entry #20943; page 5,
 *     "Add linear_qcs4w op", Constraints (3).
 *   - Flat packed weight [N, K/2], K_packed == ceil(K/2): page 3 #20945
 *     design note (a flat [N, K/2] byte array); page 5, Implementation
 *     (guards).
 *   - Nibble order: the q4gsw packer stores (odd << 4) | even, so even k sits
 *     in the LOW nibble; the qcs4w packer stores (even << 4) | odd, so even k
 *     sits in the HIGH nibble: page 5, Constraints (2).
 *   - Grouped scale index (k / group_size) * padded_N + n, per-channel scale
 *     scales[n]: page 5, Solution (Before/After vs q4gsw).
 *   - Input gradient d_x[m, k] = sum_n d_out[m, n] * dequant(W)[n, k]
 *     (contraction over N): page 3, stack entry #20943.
 *   - Binary16 scales (the q4f16_1 format of the page 4 decode kernels):
 *     each scale is widened exactly to binary32, then the layer above.
 *   - Re-quantization code = clamp(round(latent / scale), -8, 7) + 8, a
 *     zero scale giving code 8, packed into the flat [N, K/2] layout: page
 *     3, stack entries #20945 and #20946 (the round is ATen's, ties to
 *     even).
 *
 * Arithmetic: every dequantized weight (code - 8) * s is formed exactly in
 * fp64 (a 4-bit integer times a 24-bit significand fits in 53 bits); the sum
 * over k runs in ascending k in fp64, with no blocking or reordering.
 * Threads (OpenMP) only split independent output columns n; every output is
 * computed by one thread in the same order, so results do not depend on the
 * thread count.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 *
 * Pages cited by number (the texts this layer is written from):
 *   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
 *           (its stack entries #20730 ... #20801);
 *   page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
 *   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
 *           (its stack entries #20917 ... #21005);
 *   page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
 *   page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------------ */
/* Unpack: page 5 Constraints (2) (order), page 3 #20943 (code - 8).   */
/* ------------------------------------------------------------------ */

/* The raw 4-bit code (0..15) of weight (n, k). order 0: even k in the low
 * nibble (q4gsw packer); order 1: even k in the high nibble (qcs4w packer). */
static int raw_code(const uint8_t *qw, int64_t ldq, int64_t n, int64_t k,
                    int order)
{
    uint8_t byte = qw[n * ldq + k / 2];
    int k_is_even = (k % 2) == 0;
    int low = byte & 0x0F;
    int high = (byte >> 4) & 0x0F;
    if (order == 0)
        return k_is_even ? low : high;
    return k_is_even ? high : low;
}

/* Signed value c = code - 8, in [-8, 7]. */
static int signed_code(const uint8_t *qw, int64_t ldq, int64_t n, int64_t k,
                       int order)
{
    return raw_code(qw, ldq, n, k, order) - 8;
}

/* Scale of weight (n, k): grouped s[(k / gs) * lds + n]; per-channel
 * (gs == 0) s[n].  Page 5, Solution. */
static float scale_of(const float *scales, int64_t lds, int64_t gs, int64_t n,
                      int64_t k)
{
    if (gs == 0)
        return scales[n];
    return scales[(k / gs) * lds + n];
}

/* Exact fp64 dequantized weight. */
static double weight_f64(const uint8_t *qw, int64_t ldq, const float *scales,
                         int64_t lds, int64_t gs, int64_t n, int64_t k,
                         int order)
{
    return (double)signed_code(qw, ldq, n, k, order) *
           (double)scale_of(scales, lds, gs, n, k);
}

/* ------------------------------------------------------------------ */
/* IEEE binary16 round-to-nearest-even, written from the format's      */
/* definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction   */
/* bits; subnormal quantum 2^-24; largest finite 65504).               */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest binary16 (ties to even) and return its bit
 * pattern.  Only exact inputs are passed in (an fp32 value, or a 4-bit
 * integer times a binary16 value), so there is a single rounding. */
uint16_t q4o_rn_f16_bits(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00u;
    /* 65504 + half its quantum (16) is a tie between 65504 (odd fraction)
     * and 65536 (overflow), which resolves upward: everything >= 65520
     * becomes infinity. */
    if (a >= 65520.0)
        return sign | 0x7C00u;
    if (a < 0x1p-14) {
        /* subnormal (or zero): value = f * 2^-24, f in [0, 1024]; f == 1024
         * encodes the smallest normal number, 0x0400, by itself. */
        double f = rint(a * 0x1p24); /* exact scaling; rint ties to even */
        return sign | (uint16_t)f;
    }
    int e2;
    (void)frexp(a, &e2);           /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                /* unbiased exponent, -14..15 */
    double quantum = ldexp(1.0, E - 10);
    double f = rint(a / quantum);  /* in [1024, 2048] */
    if (f == 2048.0) {
        f = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7C00u;
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(f - 1024.0));
}

/* Value of a binary16 bit pattern, as a double. */
double q4o_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int E = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (E == 0x1F)
        v = f ? NAN : INFINITY;
    else if (E == 0)
        v = ldexp((double)f, -24);
    else
        v = ldexp((double)(1024 + f), E - 25);
    return sign ? -v : v;
}

/* Binary16 scales widened to binary32 (exact: every binary16 value is a
 * binary32 value).  The layer with binary16 scales is the layer of page 3
 * #20943 applied to these values.  (Page 4 runs its decode kernels on
 * q4f16_1 weights, a format the pages name without defining; it is read
 * here as 4-bit codes with binary16 group scales.) */
void q4o_f16_values(const uint16_t *h, int64_t n, float *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = (float)q4o_f16_value(h[i]);
}

void q4o_round_f16(const float *src, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = q4o_rn_f16_bits((double)src[i]);
}

/* ------------------------------------------------------------------ */
/* Stage references (bit-exact targets for the unpack / dequant stage) */
/* ------------------------------------------------------------------ */

/* codes[n * ldc + k] = q[n, k] - 8. */
void q4o_unpack_codes(const uint8_t *qw, int64_t ldq, int64_t N, int64_t K,
                      int order, int8_t *codes, int64_t ldc)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * ldc + k] = (int8_t)signed_code(qw, ldq, n, k, order);
}

/* w[n * ldw + k] = (code - 8) * s, exact, in fp64. */
void q4o_dequant_f64(const uint8_t *qw, int64_t ldq, const float *scales,
                     int64_t lds, int64_t gs, int64_t N, int64_t K, int order,
                     double *w, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w[n * ldw + k] = weight_f64(qw, ldq, scales, lds, gs, n, k, order);
}

/* fp32 dequant: the exact product (code - 8) * s rounded once to fp32. */
void q4o_dequant_f32(const uint8_t *qw, int64_t ldq, const float *scales,
                     int64_t lds, int64_t gs, int64_t N, int64_t K, int order,
                     float *w, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            w[n * ldw + k] =
                (float)weight_f64(qw, ldq, scales, lds, gs, n, k, order);
}

/* binary16 dequant: the scale is first rounded to binary16, then the exact
 * product (code - 8) * RN16(s) is rounded once to binary16 (the binary16
 * dequant multiply of page 1, stack entry #20752). */
void q4o_dequant_f16(const uint8_t *qw, int64_t ldq, const float *scales,
                     int64_t lds, int64_t gs, int64_t N, int64_t K, int order,
                     uint16_t *w, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double s16 = q4o_f16_value(
                q4o_rn_f16_bits((double)scale_of(scales, lds, gs, n, k)));
            double c = (double)signed_code(qw, ldq, n, k, order);
            w[n * ldw + k] = q4o_rn_f16_bits(c * s16);
        }
}

/* ------------------------------------------------------------------ */
/* The linear layer                                                    */
/* ------------------------------------------------------------------ */

/* One output: ascending-k fp64 sum of x[m,k] * w[n,k], plus bias[n];
 * den = sum_k |x[m,k] * w[n,k]| (the normalisation of the error metric). */
static void one_output(const float *x, int64_t ldx, const double *wrow,
                       const float *bias, int64_t m, int64_t n, int64_t K,
                       double *out, double *den)
{
    double acc = 0.0, d = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = (double)x[m * ldx + k] * wrow[k];
        acc += p;
        d += fabs(p);
    }
    if (bias)
        acc += (double)bias[n];
    *out = acc;
    *den = d;
}

/* Full output: out[m * N + n], den[m * N + n] (both [M, N], fp64). */
void q4o_linear(const float *x, int64_t ldx, const uint8_t *qw, int64_t ldq,
                const float *scales, int64_t lds, int64_t gs,
                const float *bias, int64_t M, int64_t N, int64_t K, int order,
                double *out, double *den)
{
#pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                wrow[k] = weight_f64(qw, ldq, scales, lds, gs, n, k, order);
            for (int64_t m = 0; m < M; ++m)
                one_output(x, ldx, wrow, bias, m, n, K, &out[m * N + n],
                           &den[m * N + n]);
        }
        free(wrow);
    }
}

/* Sampled outputs: out[i] = result at (ms[i], ns[i]). */
void q4o_linear_sampled(const float *x, int64_t ldx, const uint8_t *qw,
                        int64_t ldq, const float *scales, int64_t lds,
                        int64_t gs, const float *bias, int64_t K, int order,
                        int64_t P, const int64_t *ms, const int64_t *ns,
                        double *out, double *den)
{
#pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < P; ++i) {
            int64_t n = ns[i];
            for (int64_t k = 0; k < K; ++k)
                wrow[k] = weight_f64(qw, ldq, scales, lds, gs, n, k, order);
            one_output(x, ldx, wrow, bias, ms[i], n, K, &out[i], &den[i]);
        }
        free(wrow);
    }
}

/* ------------------------------------------------------------------ */
/* Input gradient: page 3, stack entry #20943                          */
/* ------------------------------------------------------------------ */

/* One input-gradient element: ascending-n fp64 sum of d_out[m,n] * w[n,k]
 * (wcol[n] = w[n,k]); den = sum_n |d_out[m,n] * w[n,k]|. */
static void one_grad(const float *dout, int64_t lddo, const double *wcol,
                     int64_t m, int64_t N, double *out, double *den)
{
    double acc = 0.0, d = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double p = (double)dout[m * lddo + n] * wcol[n];
        acc += p;
        d += fabs(p);
    }
    *out = acc;
    *den = d;
}

/* Full input gradient: dx[m * K + k], den[m * K + k] (both [M, K], fp64). */
void q4o_linear_backward(const float *dout, int64_t lddo, const uint8_t *qw,
                         int64_t ldq, const float *scales, int64_t lds,
                         int64_t gs, int64_t M, int64_t N, int64_t K,
                         int order, double *dx, double *den)
{
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t n = 0; n < N; ++n)
                wcol[n] = weight_f64(qw, ldq, scales, lds, gs, n, k, order);
            for (int64_t m = 0; m < M; ++m)
                one_grad(dout, lddo, wcol, m, N, &dx[m * K + k], &den[m * K + k]);
        }
        free(wcol);
    }
}

/* Sampled input gradient: out[i] = d_x at (ms[i], ks[i]). */
void q4o_linear_backward_sampled(const float *dout, int64_t lddo,
                                 const uint8_t *qw, int64_t ldq,
                                 const float *scales, int64_t lds, int64_t gs,
                                 int64_t N, int order, int64_t P,
                                 const int64_t *ms, const int64_t *ks,
                                 double *out, double *den)
{
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < P; ++i) {
            for (int64_t n = 0; n < N; ++n)
                wcol[n] = weight_f64(qw, ldq, scales, lds, gs, n, ks[i], order);
            one_grad(dout, lddo, wcol, ms[i], N, &out[i], &den[i]);
        }
        free(wcol);
    }
}

/* ------------------------------------------------------------------ */
/* Re-quantization and packing: page 3, stack entries #20945, #20946   */
/* ------------------------------------------------------------------ */

/* The 4-bit code of a latent weight under scale s: the quotient is formed
 * in fp32 (one IEEE division, as the fp32 buffers of the pages hold it),
 * rounded to the nearest integer with ties to even (ATen's round),
 * clamped to [-8, 7] and offset by 8.  A zero scale gives code 8 without
 * dividing; so does a quotient that is not a number (reading: NaN carries
 * no magnitude to keep). */
static int requant_code(float latent, float s)
{
    if (s == 0.0f)
        return 8;
    float q = latent / s;
    if (isnan(q))
        return 8;
    float r = nearbyintf(q); /* default rounding mode: nearest, ties to even */
    if (r < -8.0f)
        r = -8.0f;
    if (r > 7.0f)
        r = 7.0f;
    return (int)r + 8;
}

/* qw[n * ldq + b] for b < ceil(K/2): the codes of k = 2b, 2b + 1 in the
 * packer's nibble order (order 0: even k low, the q4gsw packer; order 1:
 * even k high, the qcs4w packer; page 5, Constraints (2)).  With odd K the
 * missing k = K code is 8 (a zero weight).  Bytes past ceil(K/2) in each
 * row are left as they are. */
void q4o_requant(const float *latent, int64_t ldl, const float *scales,
                 int64_t lds, int64_t gs, int64_t N, int64_t K, int order,
                 uint8_t *qw, int64_t ldq)
{
    int64_t Kp = (K + 1) / 2;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < Kp; ++b) {
            int64_t k0 = 2 * b, k1 = 2 * b + 1;
            int c0 = requant_code(latent[n * ldl + k0],
                                  scale_of(scales, lds, gs, n, k0));
            int c1 = k1 < K ? requant_code(latent[n * ldl + k1],
                                           scale_of(scales, lds, gs, n, k1))
                            : 8;
            qw[n * ldq + b] = order == 0 ? (uint8_t)((c1 << 4) | c0)
                                         : (uint8_t)((c0 << 4) | c1);
        }
}

int q4o_max_threads(void) { return omp_get_max_threads(); }
