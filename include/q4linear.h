/*
 * q4linear.h -- C ABI of the MI355X (gfx950) weight-only 4-bit linear layer.
 *
 *   out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8)  (+ bias[n])
 *
 * Operator contract (pages):
 *   - dense linear form out[m,n] = sum_k in[m,k] * weight[n,k] (+ bias[n]),
 *     bias optional: page 2, "[ExecuTorch][WebGPU] Add optimized linear_fp32
 *     op", Solution and Implementation;
 *   - dequant(W[n,k]) = (code - 8) * scale: page 3, "Add fp32 matmul ops (mm,
 *     bmm, linear)", stack entry #20943;
 *   - packed weight [N, K/2] with K_packed == ceil(K/2), grouped scales
 *     indexed (k / group_size) * padded_N + n, per-channel scales [N], nibble
 *     order of the two packers: page 5, "[ExecuTorch][WebGPU] Add linear_qcs4w
 *     op", Solution, Implementation and Constraints (2);
 *   - argument guards fail loudly, before any buffer is allocated or any
 *     work is queued: page 2, Implementation; page 5, Implementation.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named x, qw, scales, bias, out, codes, w or
 *     workspace is a DEVICE pointer owned by the caller.  The library never
 *     allocates, frees or retains device memory.
 *   - Work is queued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Results are valid once the stream reaches that point;
 *     inputs must stay alive until then.
 *   - Row pitches (ldx, ldq, lds, ldo, ldc, ldw) are in ELEMENTS of the
 *     array's type (bytes for qw and codes).  Operands need only natural
 *     element alignment; any pitch >= the row width is accepted.  A
 *     workspace must be 16-byte aligned (its kernels read and write it in
 *     16-byte pieces), else the call returns Q4_ERR_WORKSPACE.
 *   - All arguments are checked before anything is queued; on any non-OK
 *     status no memory is read or written.  Errors are return codes; no C++
 *     exception crosses this boundary.
 *   - The library keeps no state besides its loaded code objects; calls are
 *     thread-safe.  Results are deterministic: the same inputs on the same
 *     path give bit-identical outputs.
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
#ifndef Q4LINEAR_H
#define Q4LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 2

typedef int32_t q4_status;
#define Q4_OK 0
#define Q4_ERR_INVALID_ARG 1  /* NULL pointer, negative size, K <= 0, pitch
                                 below row width, unknown enum value */
#define Q4_ERR_ALIAS 2        /* out overlaps an input */
#define Q4_ERR_WORKSPACE 3    /* workspace NULL, smaller than required or
                                 not 16-byte aligned */
#define Q4_ERR_UNSUPPORTED 4  /* a valid request the library does not implement */
#define Q4_ERR_DEVICE 5       /* the HIP runtime reported a launch error */

/* Nibble order of the packed bytes (page 5, Constraints (2)). */
#define Q4_ORDER_LOW_FIRST 0  /* q4gsw packer: byte = (q[odd k] << 4) | q[even k] */
#define Q4_ORDER_HIGH_FIRST 1 /* qcs4w packer: byte = (q[even k] << 4) | q[odd k] */

/* Arithmetic of q4_linear. */
#define Q4_MATH_AUTO 0 /* M == 1: F32 GEMV.  M > 1: F16 MFMA GEMM, except
                          for very small products where the F32 low-batch
                          GEMV is faster: with K % 32 == 0 and per-channel or
                          power-of-two groups >= 32 (the few-row kernel's
                          shapes), M <= 4 with N * K <= 2^22 or M == 2 with
                          N * K <= 2^25; otherwise (power-of-two groups >= 32
                          or per-channel, K % 4 == 0) M <= 16 with
                          M * N * K <= 2^26 or M == 2 with M * N * K <= 2^30.
                          Decided on sizes alone. */
#define Q4_MATH_F32 1  /* pure fp32: f32 dequant, f32 products, f32 sums */
#define Q4_MATH_F16 2  /* binary16 operands on MFMA, fp32 accumulation;
                          never binary16 accumulation.  A = RN16(x); B =
                          RN16((q - 8) * RN16(s)), except in the few-row
                          kernel where one scale covers a whole 128-k step
                          (per-channel scales, groups >= 128): there B = q - 8
                          exactly and the scale multiplies the step's fp32
                          sum (no rounding of the product to binary16) */
#define Q4_MATH_BF16 3 /* bfloat16 operands: a valid request this library
                          does not implement; every entry point that takes
                          a math returns Q4_ERR_UNSUPPORTED for it */

/* Kernel that ran (reported through path_out). */
#define Q4_PATH_NONE 0      /* nothing queued (M == 0 or N == 0) */
#define Q4_PATH_GEMV_F32 1  /* streaming fp32 GEMV, activation rows 1..M */
#define Q4_PATH_GEMM_F16 2  /* MFMA f16 x f16 -> f32 GEMM */
#define Q4_PATH_BWD_F32 3   /* fp32 input gradient (q4_linear_backward) */
#define Q4_PATH_BWD_F16 4   /* MFMA f16 x f16 -> f32 input gradient */
#define Q4_PATH_GEMM_F16_SKINNY 5 /* binary16 operands, fp32 sums, from the
                                     few-row kernel (M <= 32; M <= 64 when
                                     N * K <= 2^25 or N >= 65536; with
                                     N <= 4096 and N * K <= 2^24 also
                                     M <= 1024 when M * N * K <= 2^31;
                                     K % 8 == 0; per-channel or
                                     power-of-two groups >= 32;
                                     dword-aligned weight rows): one
                                     launch, plus the split-K reduce where a
                                     row block's binary16 activations exceed
                                     LDS or narrow N over deep K leaves CUs
                                     without a workgroup */

/* Element type of q4_dequant's output. */
#define Q4_DTYPE_F32 0
#define Q4_DTYPE_F16 1

/*
 * q4_linear -- the layer.
 *
 *   x       float [M, ldx]        activations, ldx >= K
 *   qw      uint8 [N, ldq]        packed weights, ldq >= ceil(K / 2) bytes;
 *                                 for odd K the last byte's unused nibble is
 *                                 ignored
 *   scales  float                 group_size > 0: [ceil(K / group_size), lds],
 *                                 lds >= N, scale of (n, k) at
 *                                 (k / group_size) * lds + n (the last group
 *                                 may be partial);
 *                                 group_size == 0: per-channel [N], lds unused
 *                                 (same result as group_size >= K)
 *   bias    float [N] or NULL
 *   out     float [M, ldo]        ldo >= N; must not overlap any input
 *   nibble_order  Q4_ORDER_*
 *   math          Q4_MATH_*
 *   workspace     device scratch of at least q4_linear_workspace_bytes(...)
 *                 bytes, 16-byte aligned (may be NULL when that is 0); its
 *                 contents on entry are ignored and on exit are undefined
 *   stream        hipStream_t or NULL
 *   path_out      if not NULL, receives the Q4_PATH_* that was queued
 *
 * M == 0 or N == 0 is a valid no-op (Q4_OK, nothing queued).
 * Precision: Q4_MATH_F32 holds max |out - exact| / sum_k |x * w| to about
 * 1e-5 or better; Q4_MATH_F16 rounds x and w to binary16 (round to nearest
 * even; w = RN16((q - 8) * RN16(s))) and sums in fp32, holding the same
 * normalised error under 2e-3.  F16 operands overflow to infinity beyond
 * 65504 (IEEE); callers with such magnitudes use Q4_MATH_F32.
 */
q4_status q4_linear(const float *x, int64_t ldx, const uint8_t *qw,
                    int64_t ldq, const float *scales, int64_t lds,
                    int64_t group_size, const float *bias, float *out,
                    int64_t ldo, int64_t M, int64_t N, int64_t K,
                    int32_t nibble_order, int32_t math, void *workspace,
                    size_t workspace_bytes, void *stream, int32_t *path_out);

/*
 * q4_linear_f16_scales -- the layer with binary16 scales: the weight format
 * that the decode kernels of page 4 ("dlight.gpu.GEMV" pull request, the
 * WebLLM Llama-3.2-1B q4f16_1 GEMVs) run, read here as 4-bit codes with
 * binary16 group (or per-channel) scales.  Opt-in; the layer is unchanged
 * otherwise:
 *
 *   out[m, n] = sum_k x[m, k] * f32(s16[g(k), n]) * (q[n, k] - 8)  (+ bias[n])
 *
 * with every binary16 scale widened exactly.  Arguments, sizes, workspace,
 * math, paths and precision are those of q4_linear, except:
 *   scales  uint16 binary16 bit patterns, [ceil(K / group_size), lds] or [N],
 *           2-byte aligned (the same element indexing as q4_linear)
 * Per weight, grouped scales of 32 take 0.0625 bytes instead of 0.125.
 * Q4_MATH_F16 feeds the same MFMA operands as q4_linear does with the
 * widened scales (a binary16 scale is its own RN16).
 */
q4_status q4_linear_f16_scales(const float *x, int64_t ldx, const uint8_t *qw,
                               int64_t ldq, const uint16_t *scales,
                               int64_t lds, int64_t group_size,
                               const float *bias, float *out, int64_t ldo,
                               int64_t M, int64_t N, int64_t K,
                               int32_t nibble_order, int32_t math,
                               void *workspace, size_t workspace_bytes,
                               void *stream, int32_t *path_out);
/* Bytes of workspace q4_linear (and q4_linear_f16_scales) needs for these
 * sizes and math (0 if none).  Returns 0 as well for invalid sizes (the
 * layer then reports the error). */
size_t q4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                 int64_t group_size, int32_t math);

/*
 * q4_unpack_codes -- the signed nibble values, codes[n * ldc + k] =
 * q[n, k] - 8 in [-8, 7] (page 3 #20943; page 5 Constraints (2)), for
 * 0 <= n < N, 0 <= k < K.  codes: int8 [N, ldc], ldc >= K.  Same unpack as
 * the layer's kernels.
 */
q4_status q4_unpack_codes(const uint8_t *qw, int64_t ldq, int64_t N,
                          int64_t K, int32_t nibble_order, int8_t *codes,
                          int64_t ldc, void *stream);

/*
 * q4_linear_backward -- the input gradient of the layer,
 *
 *   dx[m, k] = sum_n dout[m, n] * (q[n, k] - 8) * s[g(k), n]
 *
 * a contraction over N of the same packed weight the forward reads (page 3,
 * "Add fp32 matmul ops (mm, bmm, linear)", stack entry #20943).
 *
 *   dout    float [M, lddo]       lddo >= N
 *   qw, ldq, scales, lds, group_size, nibble_order: as in q4_linear
 *   dx      float [M, lddx]       lddx >= K; must not overlap any input
 *   math    Q4_MATH_AUTO: F16 when M >= 16 and the group size allows it,
 *           else F32 (decided on sizes alone).
 *           Q4_MATH_F32: pure fp32 (the weight is applied
 *           as c * RN32(dout * s) when a packed word lies in one group, else
 *           as RN32(c * s); fp32 sums), path Q4_PATH_BWD_F32.
 *           Q4_MATH_F16: binary16 operands on MFMA, fp32 sums: RN16(dout)
 *           times w = RN16(c * RN16(s)) (the forward F16 path's weight
 *           operand), path Q4_PATH_BWD_F16; needs group_size == 0,
 *           group_size >= K or group_size % 8 == 0, else
 *           Q4_ERR_UNSUPPORTED.
 *   workspace     device scratch of q4_linear_backward_workspace_bytes(...)
 *                 bytes for the same math (F32: partial sums over row blocks
 *                 of the weight; F16: binary16 dout and split partials),
 *                 16-byte aligned, may be NULL when that is 0; contents on
 *                 entry ignored, on exit undefined
 *   math == Q4_MATH_BF16 returns Q4_ERR_UNSUPPORTED.
 *   stream, path_out: as in q4_linear
 *
 * Sizes are validated as in q4_linear (K > 0).  M == 0 is a no-op; N == 0
 * (an empty contraction) is Q4_ERR_INVALID_ARG.
 * Precision: max |dx - exact| / sum_n |dout * w| about 1e-5 or better for
 * F32, under 2e-3 for F16.
 */
q4_status q4_linear_backward(const float *dout, int64_t lddo, const uint8_t *qw,
                             int64_t ldq, const float *scales, int64_t lds,
                             int64_t group_size, float *dx, int64_t lddx,
                             int64_t M, int64_t N, int64_t K, int32_t nibble_order,
                             int32_t math, void *workspace, size_t workspace_bytes,
                             void *stream, int32_t *path_out);

/* Bytes of workspace q4_linear_backward needs for these sizes and math (0 if
 * none, or invalid sizes). */
size_t q4_linear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                          int64_t group_size, int32_t math);

/*
 * q4_requant -- re-quantize fp32 latent weights under fixed scales and pack
 * them into the layer's weight layout (page 3, stack entries #20945 and
 * #20946):
 *
 *   code[n, k] = clamp(round(latent[n, k] / s[g(k), n]), -8, 7) + 8
 *
 * with the quotient one IEEE fp32 division and round to nearest, ties to
 * even; a zero scale (or a quotient that is not a number) gives code 8.
 *
 *   latent  float [N, ldl]        ldl >= K
 *   scales, lds, group_size       as in q4_linear
 *   qw      uint8 [N, ldq]        ldq >= ceil(K / 2); bytes 0 .. ceil(K/2)-1
 *                                 of each row are written in nibble_order
 *                                 (odd K: the unused nibble holds code 8);
 *                                 bytes past them are left untouched; must
 *                                 not overlap latent or scales
 *   stream  hipStream_t or NULL
 *
 * N == 0 is a valid no-op.  The codes are bit-exact: equal to the oracle's
 * on every input.
 */
q4_status q4_requant(const float *latent, int64_t ldl, const float *scales,
                     int64_t lds, int64_t group_size, int64_t N, int64_t K,
                     int32_t nibble_order, uint8_t *qw, int64_t ldq, void *stream);

/*
 * q4_dequant -- the dequantized weight matrix w [N, ldw], ldw >= K:
 *   Q4_DTYPE_F32: w = RN32((q - 8) * s)          (one rounding of the exact
 *                                                 product)
 *   Q4_DTYPE_F16: w = RN16((q - 8) * RN16(s))    (the scale rounded to
 *                 binary16, then one rounding of the exact product; this is
 *                 the operand the F16 layer feeds to MFMA: the binary16
 *                 dequant multiply of page 1, stack entry #20752)
 * scales / lds / group_size as in q4_linear.  w is float* for F32 and a
 * binary16 (uint16_t bit pattern) array for F16.
 */
q4_status q4_dequant(const uint8_t *qw, int64_t ldq, const float *scales,
                     int64_t lds, int64_t group_size, int64_t N, int64_t K,
                     int32_t nibble_order, int32_t dtype, void *w,
                     int64_t ldw, void *stream);

/*
 * q4_linear_noalloc -- q4_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, checks, kernels, results and
 * Q4_PATH_* as q4_linear with the same sizes and math, without the
 * workspace arguments: the workspace is a device array inside the library,
 * Q4_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on (held from the load
 * of the library's code object until the process ends).  The caller still
 * passes x, qw, scales, bias and out.
 *
 * Runs on the current HIP device, which must be the device `stream`
 * belongs to.  The first call on a device looks up that device's array
 * (hipGetSymbolAddress); no call allocates or frees memory.
 *
 * Errors: those of q4_linear, and Q4_ERR_WORKSPACE when
 * q4_linear_workspace_bytes(M, N, K, group_size, math) exceeds
 * Q4_NOALLOC_SCRATCH_BYTES (nothing is queued); Q4_ERR_DEVICE when the
 * device or its array cannot be found.
 *
 * Concurrency: every call on one GPU uses the same array.  Calls whose work
 * overlaps in time on one GPU (different streams, or host threads queueing
 * without ordering) race on it and give undefined results; calls queued in
 * order on one stream do not.
 */
#define Q4_NOALLOC_SCRATCH_BYTES (64u << 20)
q4_status q4_linear_noalloc(const float *x, int64_t ldx, const uint8_t *qw,
                            int64_t ldq, const float *scales, int64_t lds,
                            int64_t group_size, const float *bias, float *out,
                            int64_t ldo, int64_t M, int64_t N, int64_t K,
                            int32_t nibble_order, int32_t math, void *stream,
                            int32_t *path_out);

/* Static description of a status code. */
const char *q4_status_str(q4_status status);

/* Q4_ABI_VERSION of the loaded library. */
int32_t q4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4LINEAR_H */
