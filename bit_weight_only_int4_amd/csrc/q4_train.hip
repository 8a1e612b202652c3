// q4_train.hip -- the training-side kernels of the weight-only 4-bit
// linear layer for gfx950: the input gradient and re-quantization.
//
// Input gradient (page 3, "Add fp32 matmul ops (mm, bmm, linear)", stack
// entry #20943):  d_x[m, k] = sum_n d_out[m, n] * (q[n, k] - 8) * s[g(k), n],
// a contraction over N that reads the same packed [N, K/2] weight as the
// forward, with no repacking.  Pure fp32 (binary16 only holds the exact
// integers q - 8): each lane owns 8 consecutive k (one packed word per
// row), a wave 512 k, and walks down its block of rows n, so every weight
// row is read as one 256-byte coalesced segment per wave and each weight is
// unpacked once for all of the workgroup's activation rows m.  d_out[m, n]
// is the same for every lane of a wave (a scalar load).  The 8 waves of a
// workgroup cover consecutive row blocks of the same 512 k and add their
// partial sums in LDS in wave order; when N spans several workgroups their
// partial sums go to the workspace and a second kernel adds them in a fixed
// order, so results are deterministic.
//
// Re-quantization (page 3, stack entries #20945 and #20946): code =
// clamp(round(latent / s), -8, 7) + 8 with the quotient one IEEE fp32
// division and the round to nearest, ties to even (ATen's round); a zero
// scale gives code 8 without dividing, and so does a quotient that is not a
// number.  Codes are packed into the flat [N, K/2] layout in either packer
// order (page 5, "[ExecuTorch][WebGPU] Add linear_qcs4w op", Constraints
// (2)); for odd K the unused nibble holds code 8.
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

// ---------------------------------------------------------------------------
// Re-quantization
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t requant_code(float latent, float s) {
  if (s == 0.0f) return 8u;
  const float q = latent / s;  // IEEE fp32 division (correctly rounded)
  if (q != q) return 8u;
  float r = __builtin_rintf(q);  // nearest, ties to even
  r = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  return (uint32_t)((int)r + 8);
}

// One thread per packed word (8 k, 4 bytes) of a row; grid.y strides rows.
// log2_gs >= 0: power-of-two group size; -1: any other (group_size > 0);
// group_size == 0: per-channel.
template <int ORDER>
__global__ void __launch_bounds__(256)
requant_kernel(const float* __restrict__ latent, int64_t ldl, const float* __restrict__ scales,
               int64_t lds, int64_t gs, int log2_gs, int64_t N, int64_t K,
               uint8_t* __restrict__ qw, int64_t ldq) {
  // Blocks of 2048 k wholly inside K, 16-byte aligned latents, groups of a
  // multiple of 4 k and 2-byte aligned code rows: thread t rounds the 4 k at
  // 4t and at 1024 + 4t of the block, so each wave-wide 16-byte load reads
  // 1 KiB of one row, and writes their codes as two 2-byte pieces.
  const int64_t kbl = (int64_t)blockIdx.x * 2048;
  if (kbl + 2048 <= K && (ldl % 4) == 0 && (reinterpret_cast<uintptr_t>(latent) % 16) == 0 &&
      (gs == 0 || gs % 4 == 0) && (ldq % 2) == 0 && (reinterpret_cast<uintptr_t>(qw) % 2) == 0) {
    for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
      const float* lrow = latent + n * ldl;
      uint8_t* qrow = qw + n * ldq;
      f4 a[2];
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t k = kbl + 1024 * h + 4 * threadIdx.x;
        a[h] = *reinterpret_cast<const f4*>(lrow + k);
        int64_t srow = 0;
        if (gs > 0) srow = log2_gs >= 0 ? (k >> log2_gs) : (int64_t)((uint64_t)k / (uint64_t)gs);
        sc[h] = scales[srow * lds + n];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c0 = requant_code(a[h].x, sc[h]), c1 = requant_code(a[h].y, sc[h]);
        const uint32_t c2 = requant_code(a[h].z, sc[h]), c3 = requant_code(a[h].w, sc[h]);
        const uint32_t b0 = ORDER == kLowFirst ? (c0 | (c1 << 4)) : (c1 | (c0 << 4));
        const uint32_t b1 = ORDER == kLowFirst ? (c2 | (c3 << 4)) : (c3 | (c2 << 4));
        const int64_t k = kbl + 1024 * h + 4 * threadIdx.x;
        *reinterpret_cast<uint16_t*>(qrow + k / 2) = (uint16_t)(b0 | (b1 << 8));
      }
    }
    return;
  }
  const int64_t wd = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t Kp = (K + 1) >> 1;
  if (4 * wd >= Kp) return;
  const int64_t k0 = 8 * wd;
  // whole words with 16-byte aligned latents and one group per word: two
  // 16-byte loads and one scale
  const bool fast = k0 + 8 <= K && (ldl % 4) == 0 &&
                    (reinterpret_cast<uintptr_t>(latent) % 16) == 0 && (gs == 0 || gs % 8 == 0);
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    const float* lrow = latent + n * ldl;
    uint32_t c[8];
    if (fast) {
      const f4 a = *reinterpret_cast<const f4*>(lrow + k0);
      const f4 b = *reinterpret_cast<const f4*>(lrow + k0 + 4);
      int64_t srow = 0;
      if (gs > 0) srow = log2_gs >= 0 ? (k0 >> log2_gs) : (int64_t)((uint64_t)k0 / (uint64_t)gs);
      const float sc = scales[srow * lds + n];
      c[0] = requant_code(a.x, sc); c[1] = requant_code(a.y, sc);
      c[2] = requant_code(a.z, sc); c[3] = requant_code(a.w, sc);
      c[4] = requant_code(b.x, sc); c[5] = requant_code(b.y, sc);
      c[6] = requant_code(b.z, sc); c[7] = requant_code(b.w, sc);
    }
#pragma unroll
    for (int i = 0; i < 8 && !fast; ++i) {
      const int64_t k = k0 + i;
      if (k >= K) {
        c[i] = 8u;
        continue;
      }
      int64_t srow = 0;
      if (gs > 0) srow = log2_gs >= 0 ? (k >> log2_gs) : (int64_t)((uint64_t)k / (uint64_t)gs);
      c[i] = requant_code(lrow[k], scales[srow * lds + n]);
    }
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t lo = ORDER == kLowFirst ? c[2 * b] : c[2 * b + 1];
      const uint32_t hi = ORDER == kLowFirst ? c[2 * b + 1] : c[2 * b];
      word |= (lo | (hi << 4)) << (8 * b);
    }
    uint8_t* qrow = qw + n * ldq;
    if (4 * wd + 4 <= Kp && (reinterpret_cast<uintptr_t>(qrow + 4 * wd) & 3) == 0) {
      *reinterpret_cast<uint32_t*>(qrow + 4 * wd) = word;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (4 * wd + b < Kp) qrow[4 * wd + b] = (uint8_t)(word >> (8 * b));
    }
  }
}

// ---------------------------------------------------------------------------
// Input gradient, fp32
// ---------------------------------------------------------------------------

constexpr int BW_WAVES = 8;    // waves per workgroup
constexpr int BW_CHUNK = 16;   // rows a wave loads before computing

// Workgroup (blockIdx.x, blockIdx.y, blockIdx.z): k range 512 * blockIdx.x,
// row block blockIdx.y of rows_per_wg rows (wave w takes rows_per_wg / 8 of
// them), activation rows m0 = MB * blockIdx.z .. m0 + MB - 1.
template <int ORDER, int MB, bool QA4>
__global__ void __launch_bounds__(512)
bwd_f32_kernel(const BwdParams p) {
  __shared__ float red[BW_WAVES * MB * 512];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t k0 = (int64_t)blockIdx.x * 512 + 8 * lane;
  const int64_t rows_w = p.rows_per_wg / BW_WAVES;
  const int64_t nb0 = (int64_t)blockIdx.y * p.rows_per_wg + (int64_t)w * rows_w;
  const int64_t nb1 = (nb0 + rows_w < p.N) ? nb0 + rows_w : p.N;
  const int64_t m0 = (int64_t)blockIdx.z * MB;
  const int64_t row_bytes = (p.K + 1) >> 1;
  const bool kin = k0 < p.K;
  const bool kfull = k0 + 8 <= p.K;
  // the scale row of each of this lane's 8 k (one row when a group holds
  // whole words)
  int64_t srow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = (k0 + i < p.K) ? k0 + i : p.K - 1;
    srow[i] = p.group_size == 0 ? 0
              : p.log2_gs >= 0 ? (k >> p.log2_gs)
                               : (int64_t)((uint64_t)k / (uint64_t)p.group_size);
  }
  const bool one_group = p.group_size == 0 || srow[0] == srow[7];
  const Magic mg = Magic::make();

  float acc[MB][8];
#pragma unroll
  for (int mm = 0; mm < MB; ++mm)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[mm][i] = 0.0f;

  // Interior waves (every row of the block inside N, every lane's 8 k inside
  // K, one group per packed word): all loads of a chunk issue unconditionally,
  // then the arithmetic runs without branches.
  const bool fast = QA4 && nb0 + rows_w <= p.N && (int64_t)(blockIdx.x + 1) * 512 <= p.K &&
                    (p.group_size == 0 || p.group_size % 8 == 0) && rows_w % BW_CHUNK == 0;
  if (fast) {
    const float* scol = p.scales + srow[0] * p.lds;
    for (int64_t c0 = nb0; c0 < nb1; c0 += BW_CHUNK) {
      uint32_t wv[BW_CHUNK];
      float sv[BW_CHUNK];
      float dv[MB][BW_CHUNK];
#pragma unroll
      for (int r = 0; r < BW_CHUNK; ++r) {
        wv[r] = *reinterpret_cast<const uint32_t*>(p.qw + (c0 + r) * p.ldq + (k0 >> 1));
        sv[r] = scol[c0 + r];
      }
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
#pragma unroll
        for (int r = 0; r < BW_CHUNK; ++r)
          dv[mm][r] = (m0 + mm < p.M) ? p.dout[(m0 + mm) * p.lddo + c0 + r] : 0.0f;
#pragma unroll
      for (int r = 0; r < BW_CHUNK; ++r) {
        h2 c[4];
        unpack_word(wv[r], mg, c);
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          const float ds = dv[mm][r] * sv[r];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            acc[mm][pair_k<ORDER>(pp, 0)] =
                __builtin_fmaf((float)c[pp].x, ds, acc[mm][pair_k<ORDER>(pp, 0)]);
            acc[mm][pair_k<ORDER>(pp, 1)] =
                __builtin_fmaf((float)c[pp].y, ds, acc[mm][pair_k<ORDER>(pp, 1)]);
          }
        }
      }
    }
  }

  for (int64_t c0 = nb0; c0 < nb1 && !fast; c0 += BW_CHUNK) {
    // weight words and scales of up to BW_CHUNK rows, all in flight
    uint32_t wv[BW_CHUNK];
    float sv[BW_CHUNK];
#pragma unroll
    for (int r = 0; r < BW_CHUNK; ++r) {
      const int64_t n = c0 + r;
      wv[r] = 0x88888888u;
      sv[r] = 0.0f;
      if (n < nb1 && kin) {
        const uint8_t* row = p.qw + n * p.ldq;
        if (QA4 && kfull) {
          wv[r] = *reinterpret_cast<const uint32_t*>(row + (k0 >> 1));
        } else {
          uint32_t v = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int64_t o = (k0 >> 1) + b;
            v |= (o < row_bytes ? (uint32_t)row[o] : 0x88u) << (8 * b);
          }
          wv[r] = v;
        }
        if (one_group) sv[r] = p.scales[srow[0] * p.lds + n];
      }
    }
#pragma unroll
    for (int r = 0; r < BW_CHUNK; ++r) {
      const int64_t n = c0 + r;
      if (n >= nb1) break;
      h2 c[4];
      unpack_word(wv[r], mg, c);
      if (one_group) {
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          if (m0 + mm >= p.M) break;
          // d_out[m, n] * s: one fp32 product, then exact c times it
          const float ds = p.dout[(m0 + mm) * p.lddo + n] * sv[r];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            acc[mm][pair_k<ORDER>(pp, 0)] =
                __builtin_fmaf((float)c[pp].x, ds, acc[mm][pair_k<ORDER>(pp, 0)]);
            acc[mm][pair_k<ORDER>(pp, 1)] =
                __builtin_fmaf((float)c[pp].y, ds, acc[mm][pair_k<ORDER>(pp, 1)]);
          }
        }
      } else {
        // groups narrower than a word: w = RN32(c * s) per weight
        float wgt[8];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int i = pair_k<ORDER>(pp, h);
            const float s = kin ? p.scales[srow[i] * p.lds + n] : 0.0f;
            wgt[i] = (float)(h == 0 ? c[pp].x : c[pp].y) * s;
          }
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          if (m0 + mm >= p.M) break;
          const float d = p.dout[(m0 + mm) * p.lddo + n];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[mm][i] = __builtin_fmaf(wgt[i], d, acc[mm][i]);
        }
      }
    }
  }

  // the workgroup's 8 partial sums, added in wave order
#pragma unroll
  for (int mm = 0; mm < MB; ++mm)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[(w * MB + mm) * 512 + 8 * lane + i] = acc[mm][i];
  __syncthreads();
  for (int e = threadIdx.x; e < MB * 512; e += 512) {
    const int mm = e / 512, kk = e % 512;
    const int64_t m = m0 + mm, k = (int64_t)blockIdx.x * 512 + kk;
    if (m >= p.M || k >= p.K) continue;
    float v = red[mm * 512 + kk];
    for (int ww = 1; ww < BW_WAVES; ++ww) v += red[(ww * MB + mm) * 512 + kk];
    if (p.blocks_n > 1)
      p.partial[((int64_t)blockIdx.y * p.M + m) * p.K + k] = v;
    else
      p.dx[m * p.lddx + k] = v;
  }
}

// dx[m, k] = sum over row blocks b of partial[b][m][k]: 64 elements per
// workgroup, four threads per element; thread quarter q adds blocks q, q + 4,
// q + 8, ... in order, and the four quarter sums are added in quarter order,
// so the result does not depend on timing.
__global__ void __launch_bounds__(256)
bwd_reduce_kernel(const float* __restrict__ partial, int64_t blocks, int64_t M, int64_t K,
                  float* __restrict__ dx, int64_t lddx) {
  __shared__ float red[4][64];
  const int t = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t e = (int64_t)blockIdx.x * 64 + t;
  const int64_t total = M * K;
  float v = 0.0f;
  if (e < total) {
#pragma unroll 4
    for (int64_t bb = q; bb < blocks; bb += 4) v += partial[bb * total + e];
  }
  red[q][t] = v;
  __syncthreads();
  if (q != 0 || e >= total) return;
  const int64_t m = e / K, k = e % K;
  dx[m * lddx + k] = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
}

template <int ORDER, int MB>
hipError_t launch_bwd_t(const BwdParams& p, dim3 grid, bool qa4, hipStream_t s) {
  if (qa4)
    hipLaunchKernelGGL((bwd_f32_kernel<ORDER, MB, true>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_f32_kernel<ORDER, MB, false>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace

BwdPlan plan_bwd(int64_t M, int64_t N, int64_t K) {
  BwdPlan pl{};
  pl.mb = M >= 4 ? 4 : (M >= 2 ? 2 : 1);
  pl.blocks_m = (M + pl.mb - 1) / pl.mb;
  pl.blocks_k = (K + 511) / 512;
  // rows per workgroup: at least 128, and at least 64 per activation row,
  // so the partial sums (blocks_n * M * K floats) stay at most an eighth of
  // the packed weight bytes
  int64_t rows = 128;
  while (rows < 64 * M) rows *= 2;
  // no more than N needs (rounded up to whole 16-row chunks per wave), so
  // every wave of the workgroup has rows
  const int64_t cap = ((N + BW_WAVES * BW_CHUNK - 1) / (BW_WAVES * BW_CHUNK)) * BW_WAVES * BW_CHUNK;
  if (rows > cap) rows = cap < 128 ? 128 : cap;
  pl.rows_per_wg = rows;
  pl.blocks_n = (N + rows - 1) / rows;
  return pl;
}

size_t bwd_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const BwdPlan pl = plan_bwd(M, N, K);
  return pl.blocks_n > 1 ? (size_t)pl.blocks_n * (size_t)M * (size_t)K * sizeof(float) : 0;
}

hipError_t launch_bwd_f32(const BwdParams& p0, int order, bool qa4, hipStream_t s) {
  BwdParams p = p0;
  const BwdPlan pl = plan_bwd(p.M, p.N, p.K);
  p.rows_per_wg = pl.rows_per_wg;
  p.blocks_n = pl.blocks_n;
  if (p.group_size >= p.K) p.group_size = 0;  // one group: the per-channel vector
  p.log2_gs = -1;
  if (p.group_size > 0 && (p.group_size & (p.group_size - 1)) == 0) {
    int l2 = 0;
    while ((1LL << l2) < p.group_size) ++l2;
    p.log2_gs = l2;
  }
  const dim3 grid((unsigned)pl.blocks_k, (unsigned)pl.blocks_n, (unsigned)pl.blocks_m);
  hipError_t e;
  if (order == 0)
    e = pl.mb == 4 ? launch_bwd_t<0, 4>(p, grid, qa4, s)
        : pl.mb == 2 ? launch_bwd_t<0, 2>(p, grid, qa4, s)
                     : launch_bwd_t<0, 1>(p, grid, qa4, s);
  else
    e = pl.mb == 4 ? launch_bwd_t<1, 4>(p, grid, qa4, s)
        : pl.mb == 2 ? launch_bwd_t<1, 2>(p, grid, qa4, s)
                     : launch_bwd_t<1, 1>(p, grid, qa4, s);
  if (e != hipSuccess || pl.blocks_n == 1) return e;
  const int64_t total = p.M * p.K;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((total + 63) / 64)), dim3(256), 0, s,
                     p.partial, pl.blocks_n, p.M, p.K, p.dx, p.lddx);
  return hipGetLastError();
}

hipError_t launch_requant(const float* latent, int64_t ldl, const float* scales, int64_t lds,
                          int64_t gs, int64_t N, int64_t K, int order, uint8_t* qw, int64_t ldq,
                          hipStream_t s) {
  if (gs >= K) gs = 0;  // one group: the per-channel vector
  int l2 = -1;
  if (gs > 0 && (gs & (gs - 1)) == 0) {
    l2 = 0;
    while ((1LL << l2) < gs) ++l2;
  }
  const int64_t words = ((K + 1) / 2 + 3) / 4;
  const dim3 grid((unsigned)((words + 255) / 256), (unsigned)(N < 65535 ? N : 65535));
  if (order == 0)
    hipLaunchKernelGGL(requant_kernel<0>, grid, dim3(256), 0, s, latent, ldl, scales, lds, gs,
                       l2, N, K, qw, ldq);
  else
    hipLaunchKernelGGL(requant_kernel<1>, grid, dim3(256), 0, s, latent, ldl, scales, lds, gs,
                       l2, N, K, qw, ldq);
  return hipGetLastError();
}

}  // namespace q4
