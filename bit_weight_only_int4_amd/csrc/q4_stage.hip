// q4_stage.hip -- export kernels for the unpack and dequant stages.
//
// They run the same device functions as the layer's kernels (unpack_word,
// dequant_pair_f16, splat_f16 in q4_device.h) on whole packed words, so the
// exported values are bit for bit what the GEMV and GEMM feed their
// arithmetic:
//   codes = q - 8                       (page 3, stack entry #20943)
//   F32:  w = RN32((q - 8) * s)
//   F16:  w = RN16((q - 8) * RN16(s))   (the MFMA B operand)
//
// Pages cited by number (the texts this layer is written from):
//   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
//           (its stack entries #20730 ... #20801);
//   page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
//   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
//           (its stack entries #20917 ... #21005);
//   page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
//   page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

// One thread per packed word (8 k) of one row.  Ragged rows are read byte by
// byte; bytes past the row are 0x88 and their k are not written.
template <int ORDER>
__device__ __forceinline__ uint32_t load_word(const uint8_t* row, int64_t word,
                                              int64_t row_bytes) {
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t o = 4 * word + b;
    w |= (o < row_bytes ? (uint32_t)row[o] : 0x88u) << (8 * b);
  }
  return w;
}

template <int ORDER>
__global__ void unpack_codes_kernel(const uint8_t* __restrict__ qw, int64_t ldq,
                                    int64_t N, int64_t K, int8_t* __restrict__ codes,
                                    int64_t ldc) {
  const int64_t words = (K + 7) / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * words) return;
  const int64_t n = idx / words, wd = idx % words;
  const uint8_t* row = qw + n * ldq;
  const uint32_t w = load_word<ORDER>(row, wd, (K + 1) >> 1);
  const Magic mg = Magic::make();
  h2 c[4];
  unpack_word(w, mg, c);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = 8 * wd + pair_k<ORDER>(pp, h);
      if (k < K) codes[n * ldc + k] = (int8_t)(float)(h == 0 ? c[pp].x : c[pp].y);
    }
}

template <int ORDER, int DTYPE>
__global__ void dequant_kernel(const uint8_t* __restrict__ qw, int64_t ldq,
                               const float* __restrict__ scales, int64_t lds,
                               int64_t gs, int64_t N, int64_t K, void* __restrict__ wout,
                               int64_t ldw) {
  const int64_t words = (K + 7) / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * words) return;
  const int64_t n = idx / words, wd = idx % words;
  const uint8_t* row = qw + n * ldq;
  const uint32_t w = load_word<ORDER>(row, wd, (K + 1) >> 1);
  const Magic mg = Magic::make();
  h2 c[4];
  unpack_word(w, mg, c);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int64_t k0 = 8 * wd + pair_k<ORDER>(pp, 0);
    const int64_t k1 = 8 * wd + pair_k<ORDER>(pp, 1);
    const float s0 = scales[gs == 0 ? n : (k0 < K ? k0 : K - 1) / gs * lds + n];
    const float s1 = scales[gs == 0 ? n : (k1 < K ? k1 : K - 1) / gs * lds + n];
    if (DTYPE == Q4_DTYPE_F32) {
      float* o = reinterpret_cast<float*>(wout) + n * ldw;
      if (k0 < K) o[k0] = (float)c[pp].x * s0;
      if (k1 < K) o[k1] = (float)c[pp].y * s1;
    } else {
      _Float16* o = reinterpret_cast<_Float16*>(wout) + n * ldw;
      // the GEMM applies one RN16(s) to both halves of a pair when they share
      // a group; here each half gets its own scale, which is the same value
      // whenever the halves share a group
      const h2 v0 = dequant_pair_f16(c[pp], splat_f16(s0));
      const h2 v1 = dequant_pair_f16(c[pp], splat_f16(s1));
      if (k0 < K) o[k0] = v0.x;
      if (k1 < K) o[k1] = v1.y;
    }
  }
}

}  // namespace

hipError_t launch_unpack_codes(const uint8_t* qw, int64_t ldq, int64_t N, int64_t K,
                               int order, int8_t* codes, int64_t ldc, hipStream_t s) {
  const int64_t total = N * ((K + 7) / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (order == 0)
    hipLaunchKernelGGL(unpack_codes_kernel<0>, grid, dim3(256), 0, s, qw, ldq, N, K, codes, ldc);
  else
    hipLaunchKernelGGL(unpack_codes_kernel<1>, grid, dim3(256), 0, s, qw, ldq, N, K, codes, ldc);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* qw, int64_t ldq, const float* scales, int64_t lds,
                          int64_t gs, int64_t N, int64_t K, int order, int dtype, void* w,
                          int64_t ldw, hipStream_t s) {
  const int64_t total = N * ((K + 7) / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (gs >= K) gs = 0;  // one group: scale row 0 is the per-channel vector
#define Q4_DQ(O, D)                                                                   \
  if (order == O && dtype == D) {                                                     \
    hipLaunchKernelGGL((dequant_kernel<O, D>), grid, dim3(256), 0, s, qw, ldq, scales, \
                       lds, gs, N, K, w, ldw);                                        \
    return hipGetLastError();                                                         \
  }
  Q4_DQ(0, 0) Q4_DQ(0, 1) Q4_DQ(1, 0) Q4_DQ(1, 1)
#undef Q4_DQ
  return hipErrorInvalidValue;
}

}  // namespace q4
