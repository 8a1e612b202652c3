// q4_gemv.hip -- streaming fp32 GEMV for gfx950 (the decode regime, M = 1;
// also every activation row of Q4_MATH_F32).
//
// out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8) (+ bias[n]),
// the weight-only 4-bit linear of page 3 (#20943) and page 5; at M = 1 each
// token streams the whole weight once (page 4, "Kernel level").  The pages'
// decode schedule (page 4, "Why (8, 16)": several rows per workgroup with a
// short reduction) is prior art; this kernel is laid out for wave64 and HBM3E:
//
//  * A lane owns CPL "chunks" of 32 consecutive k (16 packed bytes, read with
//    one 128-bit load).  LPR lanes share a row, so one wave-wide load covers
//    64/LPR rows x 16*LPR contiguous bytes; WK waves of a workgroup split K.
//  * The lane's 32*CPL activations are loaded once and stay in registers
//    while the workgroup walks its rows; only packed bytes and scales stream.
//  * Unpack is branch-free: four v_and_or_b32 build binary16 (1024 + q) /
//    (64 + q), one v_pk_add_f16 per pair gives the exact c = q - 8, and
//    v_fma_mix_f32 multiplies the binary16 c by the fp32 activation into an
//    fp32 sum.  No binary16 rounding touches x or the product: the path is
//    pure fp32.
//  * Grouped scales (group_size % 32 == 0): one scale per chunk, applied to
//    the chunk's partial sum.  Per-channel: applied once per output.  Any
//    other group_size: per-weight RN32(c * s), then the fp32 product.
//  * Reduction: xor-shuffles inside the LPR lanes of a row, then the WK wave
//    partials are summed in LDS in fixed order (deterministic).
//  * Split-K (grid.z > 1) writes fp32 partials to the workspace; a second
//    kernel sums them in split order and adds the bias.
#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int kMaxRowsPerBlock = 256;

enum ScaleMode : int { kPerChannel = 0, kGroup32 = 1, kGeneric = 2 };

template <bool QA4>
__device__ __forceinline__ void load_chunk(const uint8_t* row, int64_t byte0,
                                           int64_t row_bytes, bool full,
                                           uint32_t (&w)[4]) {
  if (full) {
    if (QA4) {
      const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(row + byte0);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          v |= (uint32_t)row[byte0 + 4 * d + b] << (8 * b);
        w[d] = v;
      }
    }
  } else {
    // Ragged tail: bytes past the row are replaced by 0x88 (c = 0); the
    // matching activations are zero, so they add exactly nothing.
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t o = byte0 + 4 * d + b;
        const uint32_t byte = (o < row_bytes) ? (uint32_t)row[o] : 0x88u;
        v |= byte << (8 * b);
      }
      w[d] = v;
    }
  }
}

template <int LPR, int CPL, int WK, int ORDER, int SMODE, bool QA4>
__global__ void __launch_bounds__(64 * WK)
gemv_f32_kernel(const GemvParams p) {
  constexpr int RPI = 64 / LPR;  // rows per wave-wide load
  constexpr int U = 2;           // row iterations whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rs = lane / LPR;  // row slot of this lane
  const int j = lane % LPR;   // position inside the row's lanes
  const int64_t m = blockIdx.y;
  const int z = blockIdx.z;
  const uint32_t bx = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t n0 = (int64_t)bx * p.rows_per_block;
  const int rows_here = p.rows_per_block;
  const int iters = rows_here / RPI;
  const int64_t kz0 = (int64_t)z * p.k_per_split;
  const int64_t kz1 = (kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K;
  const int64_t row_bytes = (p.K + 1) >> 1;

  __shared__ float red[WK][kMaxRowsPerBlock];

  // ---- activations of this lane's chunks, kept in registers ----
  int64_t k0[CPL];
  bool kfull[CPL], kany[CPL];
  float xr[CPL][32];
  const float* xrow = p.x + m * p.ldx;
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    k0[t] = kz0 + 32 * (int64_t)(wave * LPR * CPL + t * LPR + j);
    kfull[t] = k0[t] + 32 <= kz1;
    kany[t] = k0[t] < kz1;
    if (kfull[t]) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const f32x4_a4 xv = *reinterpret_cast<const f32x4_a4*>(xrow + k0[t] + 4 * v);
        xr[t][4 * v + 0] = xv.x; xr[t][4 * v + 1] = xv.y;
        xr[t][4 * v + 2] = xv.z; xr[t][4 * v + 3] = xv.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        xr[t][i] = (k0[t] + i < kz1) ? xrow[k0[t] + i] : 0.0f;
    }
  }

  const Magic mg = Magic::make();

  for (int it = 0; it < iters; it += U) {
    uint32_t qv[U][CPL][4];
    float sv[U][CPL];
    bool rvalid[U];
    int64_t nrow[U];
    // issue every load of the U row iterations before any arithmetic
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nrow[u] = n0 + (int64_t)(it + u) * RPI + rs;
      rvalid[u] = (it + u < iters) && (nrow[u] < p.N);
      const uint8_t* qrow = p.qw + nrow[u] * p.ldq;
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        if (rvalid[u] && kany[t]) {
          load_chunk<QA4>(qrow, k0[t] >> 1, row_bytes, kfull[t], qv[u][t]);
          if (SMODE == kGroup32)
            sv[u][t] = p.scales[(k0[t] / p.group_size) * p.lds + nrow[u]];
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d) qv[u][t][d] = 0x88888888u;
          sv[u][t] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        float part[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          h2 c[4];
          unpack_word(qv[u][t][d], mg, c);
          float a = 0.0f;
          if (SMODE == kGeneric) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int ko = 8 * d + pair_k<ORDER>(pp, h);
                int64_t g = (k0[t] + ko) / p.group_size;
                g = g < p.G - 1 ? g : p.G - 1;
                const float s = (rvalid[u] && kany[t]) ? p.scales[g * p.lds + nrow[u]] : 0.0f;
                const float w = (float)(h == 0 ? c[pp].x : c[pp].y) * s;  // RN32(c * s)
                a = __builtin_fmaf(w, xr[t][ko], a);
              }
          } else {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              a = __builtin_fmaf((float)c[pp].x, xr[t][8 * d + pair_k<ORDER>(pp, 0)], a);
              a = __builtin_fmaf((float)c[pp].y, xr[t][8 * d + pair_k<ORDER>(pp, 1)], a);
            }
          }
          part[d] = a;
        }
        const float chunk = (part[0] + part[1]) + (part[2] + part[3]);
        if (SMODE == kGroup32)
          acc = __builtin_fmaf(sv[u][t], chunk, acc);
        else
          acc += chunk;
      }
      // reduce over the LPR lanes of this row slot
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1)
        acc += __shfl_xor(acc, off, 64);
      if (j == 0 && (it + u) < iters)
        red[wave][(it + u) * RPI + rs] = acc;
    }
  }
  __syncthreads();

  for (int r = threadIdx.x; r < rows_here; r += 64 * WK) {
    const int64_t n = n0 + r;
    if (n >= p.N) continue;
    float v = red[0][r];
#pragma unroll
    for (int w = 1; w < WK; ++w) v += red[w][r];
    if (SMODE == kPerChannel) v *= p.scales[n];
    if (p.split > 1) {
      p.partial[((int64_t)z * p.M + m) * p.N + n] = v;
    } else {
      if (p.bias) v += p.bias[n];
      p.out[m * p.ldo + n] = v;
    }
  }
}

}  // namespace

__global__ void splitk_reduce_kernel(const float* __restrict__ partial,
                                     const float* __restrict__ bias,
                                     float* __restrict__ out, int64_t ldo,
                                     int64_t M, int64_t N, int split) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float v = partial[idx];
  for (int z = 1; z < split; ++z) v += partial[(int64_t)z * M * N + idx];
  if (bias) v += bias[n];
  out[m * ldo + n] = v;
}

// ---- host-side launch ----------------------------------------------------

namespace {

template <int LPR, int CPL, int WK, int ORDER, int SMODE, bool QA4>
hipError_t launch_t(const GemvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemv_f32_kernel<LPR, CPL, WK, ORDER, SMODE, QA4>), grid,
                     dim3(64 * WK), 0, s, p);
  return hipGetLastError();
}

template <int LPR, int CPL, int WK>
hipError_t launch_cfg(const GemvParams& p, dim3 grid, int order, int smode,
                      bool qa4, hipStream_t s) {
#define Q4_GEMV_CASE(O, S, A)                                        \
  if (order == O && smode == S && qa4 == A)                          \
    return launch_t<LPR, CPL, WK, O, S, A>(p, grid, s);
  Q4_GEMV_CASE(0, 0, true) Q4_GEMV_CASE(0, 1, true) Q4_GEMV_CASE(0, 2, true)
  Q4_GEMV_CASE(1, 0, true) Q4_GEMV_CASE(1, 1, true) Q4_GEMV_CASE(1, 2, true)
  Q4_GEMV_CASE(0, 0, false) Q4_GEMV_CASE(0, 1, false) Q4_GEMV_CASE(0, 2, false)
  Q4_GEMV_CASE(1, 0, false) Q4_GEMV_CASE(1, 1, false) Q4_GEMV_CASE(1, 2, false)
#undef Q4_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  GemvPlan pl{};
  // lanes per row, chunks per lane and waves per workgroup, smallest cover of K
  struct Cfg { int lpr, cpl, wk; };
  static const Cfg cfgs[] = {{8, 1, 1}, {16, 1, 4}, {32, 1, 4}, {64, 1, 4}, {64, 2, 4}};
  int ci = 4;
  for (int i = 0; i < 5; ++i) {
    const int64_t cover = (int64_t)cfgs[i].lpr * cfgs[i].cpl * cfgs[i].wk * 32;
    if (cover >= K) { ci = i; break; }
  }
  pl.cfg = ci;
  const int64_t cover = (int64_t)cfgs[ci].lpr * cfgs[ci].cpl * cfgs[ci].wk * 32;
  pl.split = (int)((K + cover - 1) / cover);
  pl.k_per_split = cover;
  const int rpi = 64 / cfgs[ci].lpr;
  // rows per workgroup: keep >= ~1024 workgroups where N allows, and at
  // least two wave-wide loads per wave
  int64_t rpb = rpi * 2;
  const int64_t target_blocks = 1024;
  while (rpb * 2 <= kMaxRowsPerBlock &&
         ((N + rpb * 2 - 1) / (rpb * 2)) * pl.split * M >= target_blocks)
    rpb *= 2;
  pl.rows_per_block = (int)rpb;
  pl.blocks_n = (N + rpb - 1) / rpb;
  (void)group_size;
  return pl;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  const GemvPlan pl = plan_gemv(M, N, K, group_size);
  return pl.split > 1 ? (size_t)pl.split * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemv(const GemvParams& p0, int order, bool qa4, hipStream_t s) {
  GemvParams p = p0;
  const GemvPlan pl = plan_gemv(p.M, p.N, p.K, p.group_size);
  p.rows_per_block = pl.rows_per_block;
  p.k_per_split = pl.k_per_split;
  p.split = pl.split;
  int smode;
  if (p.group_size == 0 || p.group_size >= p.K) smode = kPerChannel;
  else if (p.group_size % 32 == 0) smode = kGroup32;
  else smode = kGeneric;
  if (smode == kPerChannel && p.group_size != 0) {
    // one group covering all of K: the scale row 0 is a per-channel vector
    p.group_size = 0;
  }
  const dim3 grid((unsigned)pl.blocks_n, (unsigned)p.M, (unsigned)pl.split);
  hipError_t e;
  switch (pl.cfg) {
    case 0: e = launch_cfg<8, 1, 1>(p, grid, order, smode, qa4, s); break;
    case 1: e = launch_cfg<16, 1, 4>(p, grid, order, smode, qa4, s); break;
    case 2: e = launch_cfg<32, 1, 4>(p, grid, order, smode, qa4, s); break;
    case 3: e = launch_cfg<64, 1, 4>(p, grid, order, smode, qa4, s); break;
    default: e = launch_cfg<64, 2, 4>(p, grid, order, smode, qa4, s); break;
  }
  if (e != hipSuccess || pl.split == 1) return e;
  const int64_t total = p.M * p.N;
  const int threads = 256;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + threads - 1) / threads)),
                     dim3(threads), 0, s, p.partial, p.bias, p.out, p.ldo, p.M, p.N,
                     p.split);
  return hipGetLastError();
}

}  // namespace q4
