// q4_abi.hip -- the C ABI (include/q4linear.h): argument checks, regime
// selection and launches on the caller's stream.
//
// Regime (page 1, stack entry #20730: M > 1 prefill GEMM; page 4: M = 1 decode
// GEMV): Q4_MATH_AUTO runs the fp32 GEMV for M == 1 and for small batches
// (resolve_math) and the binary16 MFMA GEMM otherwise.  There is no
// fall-back ladder: each request runs the kernel its math names, with ragged
// shapes handled inside the kernel.
//
// Every check runs before anything is queued: the pages' guards reject bad
// arguments loudly and before any buffer is allocated (page 2, "[ExecuTorch]
// [WebGPU] Add optimized linear_fp32 op", Implementation; page 5, "[ExecuTorch]
// [WebGPU] Add linear_qcs4w op", Implementation).
//
// Pages cited by number (the texts this layer is written from):
//   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
//           (its stack entries #20730 ... #20801);
//   page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
//   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
//           (its stack entries #20917 ... #21005);
//   page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
//   page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_kernels.h"
#include "q4linear.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t rows, int64_t pitch, int64_t width, int64_t elem) {
  if (!p || rows <= 0 || width <= 0) return Range{0, 0};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(((rows - 1) * pitch + width) * elem)};
}

bool overlap(Range a, Range b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// sizes representable in the kernels' index arithmetic
constexpr int64_t kMaxDim = (int64_t)1 << 31;

// Q4_MATH_AUTO: fp32 for M == 1 (the GEMV); binary16 MFMA for M > 1, except
// for the few very small products where the fp32 low-batch GEMV is faster.
// Measured on MI355X over the Llama-shaped projections (rotating weight
// copies, graph-launched): where the few-row MFMA kernel takes the shape
// (M <= 32, K % 32 == 0, per-channel or power-of-two groups >= 32) it wins
// from M = 3 up except at N * K = 2^22 (M <= 4), and at M = 2 from
// N * K > 2^25 (the 8B gate/up and down projections, the lm_head).  Where it
// does not take the shape the tiled GEMM's three launches cost 10-25 us at
// small M, and the fp32 kernel stays the faster for M <= 16 with
// M * N * K <= 2^26 and for M == 2 up to M * N * K = 2^30.  Sizes only, so
// the workspace query and the call agree.
int32_t resolve_math(int32_t math, int64_t M, int64_t N, int64_t K, int64_t group_size) {
  if (math != Q4_MATH_AUTO) return math;
  if (M == 1) return Q4_MATH_F32;
  const bool perch = group_size == 0 || group_size >= K;
  const bool pow2 = (group_size & (group_size - 1)) == 0 && group_size >= 32;
  const bool staged = perch || (pow2 && group_size <= 2048);
  const double nk = (double)N * (double)K;
  if (M <= 32 && K % 32 == 0 && K >= 128 && (perch || pow2)) {
    const bool tiny = (M <= 4 && nk <= (double)(1LL << 22)) ||
                      (M == 2 && nk <= (double)(1LL << 25));
    return staged && tiny ? Q4_MATH_F32 : Q4_MATH_F16;
  }
  const double mnk = (double)M * nk;
  const bool few = (M <= 16 && mnk <= (double)(1LL << 26)) ||
                   (M <= 2 && mnk <= (double)(1LL << 30));
  if (staged && K % 4 == 0 && few) return Q4_MATH_F32;
  return Q4_MATH_F16;
}

// The MFMA input gradient applies one scale per packed word: per-channel
// scales, or groups that are whole words.
bool bwd_mfma_groups(int64_t K, int64_t group_size) {
  return group_size == 0 || group_size >= K || group_size % 8 == 0;
}

// Arithmetic of the input gradient.  Q4_MATH_AUTO, as for the forward:
// fp32 for few activation rows, binary16 operands on MFMA from 16 rows on
// (measured faster there on MI355X, 7x at 512 rows) when the groups allow
// it.  Sizes only, so the workspace query and the call agree.
int32_t resolve_bwd_math(int32_t math, int64_t M, int64_t N, int64_t K, int64_t group_size) {
  (void)N;
  if (math != Q4_MATH_AUTO) return math;
  return (M >= 16 && bwd_mfma_groups(K, group_size)) ? Q4_MATH_F16 : Q4_MATH_F32;
}

}  // namespace

extern "C" {

int32_t q4_abi_version(void) { return Q4_ABI_VERSION; }

const char* q4_status_str(q4_status st) {
  switch (st) {
    case Q4_OK: return "ok";
    case Q4_ERR_INVALID_ARG: return "invalid argument";
    case Q4_ERR_ALIAS: return "output overlaps an input";
    case Q4_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4_ERR_UNSUPPORTED: return "unsupported request";
    case Q4_ERR_DEVICE: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t q4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size,
                                 int32_t math) {
  if (M <= 0 || N <= 0 || K <= 0 || group_size < 0 || M >= kMaxDim || N >= kMaxDim ||
      K >= kMaxDim)
    return 0;
  const int32_t m = resolve_math(math, M, N, K, group_size);
  if (m == Q4_MATH_F32) return q4::gemv_workspace_bytes(M, N, K, group_size);
  if (m == Q4_MATH_F16) return q4::gemm_workspace_bytes(M, N, K, group_size);
  return 0;
}

}  // extern "C"

namespace {

// The layer, for fp32 scales (s32) or binary16 scales (s16); exactly one is
// given.  Every check runs before anything is queued.
q4_status linear_impl(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldq,
                      const float* s32, const _Float16* s16, int64_t lds, int64_t group_size,
                      const float* bias, float* out, int64_t ldo, int64_t M, int64_t N,
                      int64_t K, int32_t nibble_order, int32_t math, void* workspace,
                      size_t workspace_bytes, void* stream, int32_t* path_out) {
  if (path_out) *path_out = Q4_PATH_NONE;
  // ---- scalar checks ----
  if (M < 0 || N < 0 || K <= 0 || group_size < 0) return Q4_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return Q4_ERR_INVALID_ARG;
  if (nibble_order != Q4_ORDER_LOW_FIRST && nibble_order != Q4_ORDER_HIGH_FIRST)
    return Q4_ERR_INVALID_ARG;
  if (math < Q4_MATH_AUTO || math > Q4_MATH_BF16) return Q4_ERR_INVALID_ARG;
  const int64_t Kp = (K + 1) / 2;
  const int64_t G = group_size == 0 ? 1 : (K + group_size - 1) / group_size;
  if (ldx < K || ldq < Kp || ldo < N) return Q4_ERR_INVALID_ARG;
  if (group_size > 0 && lds < N) return Q4_ERR_INVALID_ARG;
  // a valid request this library has no kernels for: never a silent
  // substitute
  if (math == Q4_MATH_BF16) return Q4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return Q4_OK;
  // ---- pointer checks ----
  const void* scales = s16 ? (const void*)s16 : (const void*)s32;
  const int64_t selem = s16 ? 2 : 4;
  if (!x || !qw || !scales || !out) return Q4_ERR_INVALID_ARG;
  if (!aligned(x, 4) || !aligned(scales, selem) || !aligned(out, 4) ||
      (bias && !aligned(bias, 4)))
    return Q4_ERR_INVALID_ARG;
  const Range r_out = span(out, M, ldo, N, 4);
  const Range r_x = span(x, M, ldx, K, 4);
  const Range r_q = span(qw, N, ldq, Kp, 1);
  const Range r_s =
      group_size == 0 ? span(scales, 1, N, N, selem) : span(scales, G, lds, N, selem);
  const Range r_b = span(bias, 1, N, N, 4);
  if (overlap(r_out, r_x) || overlap(r_out, r_q) || overlap(r_out, r_s) ||
      overlap(r_out, r_b))
    return Q4_ERR_ALIAS;
  const int32_t m = resolve_math(math, M, N, K, group_size);
  const size_t need = q4_linear_workspace_bytes(M, N, K, group_size, m);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return Q4_ERR_WORKSPACE;
    const Range r_w{reinterpret_cast<uintptr_t>(workspace),
                    reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(r_w, r_out) || overlap(r_w, r_x) || overlap(r_w, r_q) ||
        overlap(r_w, r_s) || overlap(r_w, r_b))
      return Q4_ERR_ALIAS;
  }
  // 16-byte weight loads need dword-aligned rows; otherwise bytes are read
  // one at a time
  const bool qa4 = aligned(qw, 4) && (ldq % 4 == 0);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (m == Q4_MATH_F32) {
    // one activation row per grid row; grid.y is at most 65535
    const int64_t mchunk = 65535;
    e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += mchunk) {
      q4::GemvParams p{};
      const int64_t mm = (M - m0 < mchunk) ? M - m0 : mchunk;
      p.x = x + m0 * ldx; p.ldx = ldx; p.qw = qw; p.ldq = ldq;
      p.scales = s32; p.scales16 = s16; p.lds = lds; p.group_size = group_size; p.G = G;
      p.bias = bias; p.out = out + m0 * ldo; p.ldo = ldo;
      p.partial = reinterpret_cast<float*>(workspace);
      p.M = mm; p.N = N; p.K = K;
      e = q4::launch_gemv(p, nibble_order, qa4, s);
    }
    if (path_out) *path_out = Q4_PATH_GEMV_F32;
  } else {
    q4::GemmParams p{};
    p.x = x; p.ldx = ldx; p.qw = qw; p.ldq = ldq;
    p.scales = s32; p.scales16 = s16; p.lds = lds; p.group_size = group_size; p.G = G;
    p.bias = bias; p.out = out; p.ldo = ldo;
    p.M = M; p.N = N; p.K = K;
    bool skinny = false;
    e = q4::launch_gemm(p, nibble_order, qa4, workspace, s, &skinny);
    if (path_out) *path_out = skinny ? Q4_PATH_GEMM_F16_SKINNY : Q4_PATH_GEMM_F16;
  }
  return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE;
}

}  // namespace

extern "C" {

q4_status q4_linear(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldq,
                    const float* scales, int64_t lds, int64_t group_size, const float* bias,
                    float* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                    int32_t nibble_order, int32_t math, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t* path_out) {
  return linear_impl(x, ldx, qw, ldq, scales, nullptr, lds, group_size, bias, out, ldo, M, N,
                     K, nibble_order, math, workspace, workspace_bytes, stream, path_out);
}

q4_status q4_linear_f16_scales(const float* x, int64_t ldx, const uint8_t* qw, int64_t ldq,
                               const uint16_t* scales, int64_t lds, int64_t group_size,
                               const float* bias, float* out, int64_t ldo, int64_t M,
                               int64_t N, int64_t K, int32_t nibble_order, int32_t math,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int32_t* path_out) {
  return linear_impl(x, ldx, qw, ldq, nullptr, reinterpret_cast<const _Float16*>(scales), lds,
                     group_size, bias, out, ldo, M, N, K, nibble_order, math, workspace,
                     workspace_bytes, stream, path_out);
}

size_t q4_linear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size,
                                          int32_t math) {
  if (M <= 0 || N <= 0 || K <= 0 || group_size < 0 || M >= kMaxDim || N >= kMaxDim ||
      K >= kMaxDim)
    return 0;
  const int32_t m = resolve_bwd_math(math, M, N, K, group_size);
  if (m == Q4_MATH_F32) return q4::bwd_workspace_bytes(M, N, K);
  if (m == Q4_MATH_F16) return q4::bwd_mfma_workspace_bytes(M, N, K);
  return 0;
}

q4_status q4_linear_backward(const float* dout, int64_t lddo, const uint8_t* qw, int64_t ldq,
                             const float* scales, int64_t lds, int64_t group_size, float* dx,
                             int64_t lddx, int64_t M, int64_t N, int64_t K,
                             int32_t nibble_order, int32_t math, void* workspace,
                             size_t workspace_bytes, void* stream, int32_t* path_out) {
  if (path_out) *path_out = Q4_PATH_NONE;
  if (M < 0 || N <= 0 || K <= 0 || group_size < 0) return Q4_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return Q4_ERR_INVALID_ARG;
  if (nibble_order != Q4_ORDER_LOW_FIRST && nibble_order != Q4_ORDER_HIGH_FIRST)
    return Q4_ERR_INVALID_ARG;
  if (math < Q4_MATH_AUTO || math > Q4_MATH_BF16) return Q4_ERR_INVALID_ARG;
  const int64_t Kp = (K + 1) / 2;
  const int64_t G = group_size == 0 ? 1 : (K + group_size - 1) / group_size;
  if (lddo < N || ldq < Kp || lddx < K) return Q4_ERR_INVALID_ARG;
  if (group_size > 0 && lds < N) return Q4_ERR_INVALID_ARG;
  if (math == Q4_MATH_BF16) return Q4_ERR_UNSUPPORTED;
  const int32_t m = resolve_bwd_math(math, M, N, K, group_size);
  if (m == Q4_MATH_F16 && !bwd_mfma_groups(K, group_size)) return Q4_ERR_UNSUPPORTED;
  if (M == 0) return Q4_OK;
  if (!dout || !qw || !scales || !dx) return Q4_ERR_INVALID_ARG;
  if (!aligned(dout, 4) || !aligned(scales, 4) || !aligned(dx, 4)) return Q4_ERR_INVALID_ARG;
  const Range r_dx = span(dx, M, lddx, K, 4);
  const Range r_do = span(dout, M, lddo, N, 4);
  const Range r_q = span(qw, N, ldq, Kp, 1);
  const Range r_s = group_size == 0 ? span(scales, 1, N, N, 4) : span(scales, G, lds, N, 4);
  if (overlap(r_dx, r_do) || overlap(r_dx, r_q) || overlap(r_dx, r_s)) return Q4_ERR_ALIAS;
  const size_t need = q4_linear_backward_workspace_bytes(M, N, K, group_size, m);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return Q4_ERR_WORKSPACE;
    const Range r_w{reinterpret_cast<uintptr_t>(workspace),
                    reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(r_w, r_dx) || overlap(r_w, r_do) || overlap(r_w, r_q) || overlap(r_w, r_s))
      return Q4_ERR_ALIAS;
  }
  q4::BwdParams p{};
  p.dout = dout; p.lddo = lddo; p.qw = qw; p.ldq = ldq;
  p.scales = scales; p.lds = lds; p.group_size = group_size;
  p.dx = dx; p.lddx = lddx; p.partial = reinterpret_cast<float*>(workspace);
  p.M = M; p.N = N; p.K = K;
  const bool qa4 = aligned(qw, 4) && (ldq % 4 == 0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (m == Q4_MATH_F16) {
    e = q4::launch_bwd_mfma(p, nibble_order, qa4, workspace, st);
    if (path_out) *path_out = Q4_PATH_BWD_F16;
  } else {
    e = q4::launch_bwd_f32(p, nibble_order, qa4, st);
    if (path_out) *path_out = Q4_PATH_BWD_F32;
  }
  return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE;
}

q4_status q4_requant(const float* latent, int64_t ldl, const float* scales, int64_t lds,
                     int64_t group_size, int64_t N, int64_t K, int32_t nibble_order,
                     uint8_t* qw, int64_t ldq, void* stream) {
  if (N < 0 || K <= 0 || group_size < 0 || N >= kMaxDim || K >= kMaxDim)
    return Q4_ERR_INVALID_ARG;
  if (nibble_order != Q4_ORDER_LOW_FIRST && nibble_order != Q4_ORDER_HIGH_FIRST)
    return Q4_ERR_INVALID_ARG;
  const int64_t Kp = (K + 1) / 2;
  const int64_t G = group_size == 0 ? 1 : (K + group_size - 1) / group_size;
  if (ldl < K || ldq < Kp) return Q4_ERR_INVALID_ARG;
  if (group_size > 0 && lds < N) return Q4_ERR_INVALID_ARG;
  if (N == 0) return Q4_OK;
  if (!latent || !scales || !qw) return Q4_ERR_INVALID_ARG;
  if (!aligned(latent, 4) || !aligned(scales, 4)) return Q4_ERR_INVALID_ARG;
  const Range r_q = span(qw, N, ldq, Kp, 1);
  const Range r_s = group_size == 0 ? span(scales, 1, N, N, 4) : span(scales, G, lds, N, 4);
  if (overlap(r_q, span(latent, N, ldl, K, 4)) || overlap(r_q, r_s)) return Q4_ERR_ALIAS;
  const hipError_t e = q4::launch_requant(latent, ldl, scales, lds, group_size, N, K,
                                          nibble_order, qw, ldq,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE;
}

q4_status q4_unpack_codes(const uint8_t* qw, int64_t ldq, int64_t N, int64_t K,
                          int32_t nibble_order, int8_t* codes, int64_t ldc, void* stream) {
  if (N < 0 || K <= 0 || N >= kMaxDim || K >= kMaxDim) return Q4_ERR_INVALID_ARG;
  if (nibble_order != Q4_ORDER_LOW_FIRST && nibble_order != Q4_ORDER_HIGH_FIRST)
    return Q4_ERR_INVALID_ARG;
  const int64_t Kp = (K + 1) / 2;
  if (ldq < Kp || ldc < K) return Q4_ERR_INVALID_ARG;
  if (N == 0) return Q4_OK;
  if (!qw || !codes) return Q4_ERR_INVALID_ARG;
  if (overlap(span(codes, N, ldc, K, 1), span(qw, N, ldq, Kp, 1))) return Q4_ERR_ALIAS;
  const hipError_t e = q4::launch_unpack_codes(qw, ldq, N, K, nibble_order, codes, ldc,
                                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE;
}

q4_status q4_dequant(const uint8_t* qw, int64_t ldq, const float* scales, int64_t lds,
                     int64_t group_size, int64_t N, int64_t K, int32_t nibble_order,
                     int32_t dtype, void* w, int64_t ldw, void* stream) {
  if (N < 0 || K <= 0 || group_size < 0 || N >= kMaxDim || K >= kMaxDim)
    return Q4_ERR_INVALID_ARG;
  if (nibble_order != Q4_ORDER_LOW_FIRST && nibble_order != Q4_ORDER_HIGH_FIRST)
    return Q4_ERR_INVALID_ARG;
  if (dtype != Q4_DTYPE_F32 && dtype != Q4_DTYPE_F16) return Q4_ERR_INVALID_ARG;
  const int64_t Kp = (K + 1) / 2;
  const int64_t G = group_size == 0 ? 1 : (K + group_size - 1) / group_size;
  if (ldq < Kp || ldw < K) return Q4_ERR_INVALID_ARG;
  if (group_size > 0 && lds < N) return Q4_ERR_INVALID_ARG;
  if (N == 0) return Q4_OK;
  if (!qw || !scales || !w) return Q4_ERR_INVALID_ARG;
  const int64_t esz = dtype == Q4_DTYPE_F32 ? 4 : 2;
  if (!aligned(scales, 4) || !aligned(w, (uintptr_t)esz)) return Q4_ERR_INVALID_ARG;
  const Range r_w = span(w, N, ldw, K, esz);
  const Range r_s = group_size == 0 ? span(scales, 1, N, N, 4) : span(scales, G, lds, N, 4);
  if (overlap(r_w, span(qw, N, ldq, Kp, 1)) || overlap(r_w, r_s)) return Q4_ERR_ALIAS;
  const hipError_t e = q4::launch_dequant(qw, ldq, scales, lds, group_size, N, K,
                                          nibble_order, dtype, w, ldw,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE;
}

}  // extern "C"
