// q4_gemm.hip -- prefill GEMM for gfx950 (M > 1): binary16 operands on MFMA,
// fp32 accumulation.
//
// out[m, n] = sum_k RN16(x[m, k]) * RN16((q[n, k] - 8) * RN16(s[g(k), n]))
//             (+ bias[n]), summed in fp32.
// Precision recipe: binary16 operands, fp32 accumulator, never binary16
// accumulation (page 1, stack entry #20752, "f16 multiply / f32 accumulate");
// every packed word and scale crosses into the chip once per tile and is
// unpacked once (page 1, stack entry #20798, the packed-word-dequant
// staging).  The pages' 64x64 / 256-thread WGSL tile is prior art only.
//
// Layout on gfx950 (wave64, v_mfma_f32_16x16x32_f16):
//  * A workgroup (4 waves) owns a BM x (4*WN) output tile; wave w owns the
//    columns [w*WN, (w+1)*WN) for all BM rows, so every dequantized weight is
//    produced exactly once per tile.
//  * K advances in steps of 128.  Activations of the step (BM x 128 fp32)
//    are read from global memory, rounded to binary16 and written into a
//    double-buffered LDS tile, shared by the four waves.
//  * Weights do not pass through LDS: lane (j, b) of a wave reads the 16
//    packed bytes holding k = 32b .. 32b+31 of column j of each 16-column
//    subtile (one 128-bit load), unpacks them with v_and_or_b32 /
//    v_pk_add_f16 and scales them with v_pk_mul_f16 into MFMA B fragments.
//    Word t of those 16 bytes feeds MFMA t of the step.
//  * The k order inside each 8-element fragment follows the nibble order of
//    the packed word; the activation tile is stored with the same
//    permutation, so A and B fragments pair up k for k.
//  * Ragged M, N and K are masked in-kernel (zero activations, 0x88 bytes,
//    predicated stores); no fall-back kernel.
//  * Split-K (grid.z > 1) writes fp32 partials to the workspace; the shared
//    reduce kernel sums them in split order and adds the bias.
#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int KS = 128;        // k per pipeline step
constexpr int APITCH = KS + 8; // LDS row pitch in halves (bank-conflict pad)

enum ScaleMode : int { kPerChannel = 0, kGroup32 = 1, kGroup8 = 2, kGeneric = 3 };

template <int BM, int WN, int ORDER, int SMODE, bool QA4>
__global__ void __launch_bounds__(256)
gemm_f16_kernel(const GemmParams p) {
  constexpr int NSUB = WN / 16;   // 16-column subtiles per wave
  constexpr int MSUB = BM / 16;   // 16-row subtiles
  constexpr int BN = 4 * WN;
  constexpr int UNITS = BM * KS / 8;          // 8-element activation units per step
  constexpr int UPT = UNITS / 256;            // units per thread
  static_assert(UNITS % 256 == 0, "tile");

  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * APITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lj = lane & 15;   // column (B) / row (A) inside a 16-subtile
  const int lb = lane >> 4;   // k block of the lane

  const uint32_t tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tm = (int)(tile % (uint32_t)p.tiles_m);
  const int tn = (int)(tile / (uint32_t)p.tiles_m);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t nw0 = (int64_t)tn * BN + (int64_t)wave * WN;
  const int z = blockIdx.z;
  const int64_t kz0 = (int64_t)z * p.k_per_split;
  const int64_t kz1 = (kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K;
  const int64_t row_bytes = (p.K + 1) >> 1;
  const int nsteps = (int)((kz1 - kz0 + KS - 1) / KS);

  // ---- per-lane B columns ----
  int64_t ncol[NSUB];
  bool nvalid[NSUB];
  const uint8_t* qrow[NSUB];
  h2 s16c[NSUB];  // per-channel scale, rounded once
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    ncol[s] = nw0 + s * 16 + lj;
    nvalid[s] = ncol[s] < p.N;
    qrow[s] = p.qw + (nvalid[s] ? ncol[s] : 0) * p.ldq;
    if (SMODE == kPerChannel)
      s16c[s] = splat_f16(nvalid[s] ? p.scales[ncol[s]] : 0.0f);
  }

  // ---- activation staging: global fp32 -> registers ----
  float4 xa[UPT][2];
  auto load_a = [&](int step) {
    const int64_t kb = kz0 + (int64_t)step * KS;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * 256;
      const int r = unit / (KS / 8);
      const int g8 = unit % (KS / 8);
      const int64_t row = m0 + r;
      const int64_t k = kb + 8 * g8;
      const float* src = p.x + row * p.ldx + k;
      if (row < p.M && k + 8 <= kz1) {
        const f32x4_a4 v0 = *reinterpret_cast<const f32x4_a4*>(src);
        const f32x4_a4 v1 = *reinterpret_cast<const f32x4_a4*>(src + 4);
        xa[u][0] = make_float4(v0.x, v0.y, v0.z, v0.w);
        xa[u][1] = make_float4(v1.x, v1.y, v1.z, v1.w);
      } else {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          t[i] = (row < p.M && k + i < kz1) ? src[i] : 0.0f;
        xa[u][0] = make_float4(t[0], t[1], t[2], t[3]);
        xa[u][1] = make_float4(t[4], t[5], t[6], t[7]);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * 256;
      const int r = unit / (KS / 8);
      const int g8 = unit % (KS / 8);
      const float v[8] = {xa[u][0].x, xa[u][0].y, xa[u][0].z, xa[u][0].w,
                          xa[u][1].x, xa[u][1].y, xa[u][1].z, xa[u][1].w};
      h8 h;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl)
        h[sl] = (_Float16)v[pair_k<ORDER>(sl >> 1, sl & 1)];  // RN16, permuted
      *reinterpret_cast<h8*>(&As[buf][r * APITCH + 8 * g8]) = h;
    }
  };

  // ---- weight chunks: 16 packed bytes per lane per subtile ----
  uint32_t qc[NSUB][4];
  float sc[NSUB][4];  // kGroup32: [s][0]; kGroup8: per word
  auto load_b = [&](int step) {
    const int64_t kb = kz0 + (int64_t)step * KS + 32 * lb;
    const bool full = kb + 32 <= kz1;
    const bool any = kb < kz1;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (nvalid[s] && any) {
        const uint8_t* row = qrow[s];
        const int64_t byte0 = kb >> 1;
        if (full && QA4) {
          const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(row + byte0);
          qc[s][0] = v.x; qc[s][1] = v.y; qc[s][2] = v.z; qc[s][3] = v.w;
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int64_t o = byte0 + 4 * d + b;
              // bytes past the row hold no k < K; their activations are 0
              const bool in = full || o < row_bytes;
              w |= (in ? (uint32_t)row[o] : 0x88u) << (8 * b);
            }
            qc[s][d] = w;
          }
        }
        if (SMODE == kGroup32) {
          sc[s][0] = p.scales[(kb / p.group_size) * p.lds + ncol[s]];
        } else if (SMODE == kGroup8) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            int64_t g = (kb + 8 * d) / p.group_size;
            g = g < p.G - 1 ? g : p.G - 1;
            sc[s][d] = p.scales[g * p.lds + ncol[s]];
          }
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) { qc[s][d] = 0x88888888u; sc[s][d] = 0.0f; }
      }
    }
  };

  f4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[i][s] = f4{0.f, 0.f, 0.f, 0.f};

  const Magic mg = Magic::make();

  if (nsteps > 0) {
    load_a(0);
    load_b(0);
    store_a(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    uint32_t qcur[NSUB][4];
    float scur[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int d = 0; d < 4; ++d) { qcur[s][d] = qc[s][d]; scur[s][d] = sc[s][d]; }
    const int64_t kb_lane = kz0 + (int64_t)step * KS + 32 * lb;
    const bool more = step + 1 < nsteps;
    if (more) {
      load_a(step + 1);
      load_b(step + 1);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8 bf[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        h2 c[4];
        unpack_word(qcur[s][t], mg, c);
        h2 w[4];
        if (SMODE == kGeneric) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              int64_t g = (kb_lane + 8 * t + pair_k<ORDER>(pp, h)) / p.group_size;
              g = g < p.G - 1 ? g : p.G - 1;
              const float sv = nvalid[s] ? p.scales[g * p.lds + ncol[s]] : 0.0f;
              const _Float16 s16 = (_Float16)sv;
              const _Float16 cc = h == 0 ? c[pp].x : c[pp].y;
              if (h == 0) w[pp].x = cc * s16; else w[pp].y = cc * s16;
            }
        } else {
          h2 s16;
          if (SMODE == kPerChannel) s16 = s16c[s];
          else if (SMODE == kGroup32) s16 = splat_f16(scur[s][0]);
          else s16 = splat_f16(scur[s][t]);
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) w[pp] = dequant_pair_f16(c[pp], s16);
        }
        bf[s] = h8{w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
      }
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        const h8 af = *reinterpret_cast<const h8*>(
            &As[buf][(i * 16 + lj) * APITCH + 32 * lb + 8 * t]);
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[s], acc[i][s], 0, 0, 0);
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[4*lb + r][lj] of each 16x16 subtile ----
  float bcol[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
    bcol[s] = (p.split == 1 && p.bias && nvalid[s]) ? p.bias[ncol[s]] : 0.0f;
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + i * 16 + 4 * lb + r;
      if (row >= p.M) continue;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (!nvalid[s]) continue;
        const float v = acc[i][s][r];
        if (p.split > 1)
          p.partial[((int64_t)z * p.M + row) * p.N + ncol[s]] = v;
        else
          p.out[row * p.ldo + ncol[s]] = v + bcol[s];
      }
    }
}

template <int BM, int WN, int ORDER, int SMODE, bool QA4>
hipError_t launch_t(const GemmParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f16_kernel<BM, WN, ORDER, SMODE, QA4>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BM, int WN>
hipError_t launch_cfg(const GemmParams& p, dim3 grid, int order, int smode, bool qa4,
                      hipStream_t s) {
#define Q4_GEMM_CASE(O, S, A) \
  if (order == O && smode == S && qa4 == A) return launch_t<BM, WN, O, S, A>(p, grid, s);
  Q4_GEMM_CASE(0, 0, true) Q4_GEMM_CASE(0, 1, true) Q4_GEMM_CASE(0, 2, true) Q4_GEMM_CASE(0, 3, true)
  Q4_GEMM_CASE(1, 0, true) Q4_GEMM_CASE(1, 1, true) Q4_GEMM_CASE(1, 2, true) Q4_GEMM_CASE(1, 3, true)
  Q4_GEMM_CASE(0, 0, false) Q4_GEMM_CASE(0, 1, false) Q4_GEMM_CASE(0, 2, false) Q4_GEMM_CASE(0, 3, false)
  Q4_GEMM_CASE(1, 0, false) Q4_GEMM_CASE(1, 1, false) Q4_GEMM_CASE(1, 2, false) Q4_GEMM_CASE(1, 3, false)
#undef Q4_GEMM_CASE
  return hipErrorInvalidValue;
}

struct Cfg { int bm, wn; };
constexpr Cfg kCfgs[] = {{64, 32}, {128, 64}};

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  (void)group_size;
  GemmPlan pl{};
  pl.cfg = (M <= 64) ? 0 : 1;
  const int bm = kCfgs[pl.cfg].bm, bn = 4 * kCfgs[pl.cfg].wn;
  pl.tiles_m = (int)((M + bm - 1) / bm);
  pl.tiles_n = (int)((N + bn - 1) / bn);
  const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
  const int64_t ksteps = (K + KS - 1) / KS;
  // split K while the grid is under ~one workgroup per CU and every split
  // keeps at least 4 steps
  int split = 1;
  while (tiles * split * 2 <= 256 && ksteps / (split * 2) >= 4) split *= 2;
  pl.split = split;
  pl.k_per_split = ((ksteps + split - 1) / split) * KS;
  pl.split = (int)((K + pl.k_per_split - 1) / pl.k_per_split);
  return pl;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  const GemmPlan pl = plan_gemm(M, N, K, group_size);
  return pl.split > 1 ? (size_t)pl.split * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmParams& p0, int order, bool qa4, hipStream_t s) {
  GemmParams p = p0;
  const GemmPlan pl = plan_gemm(p.M, p.N, p.K, p.group_size);
  p.split = pl.split;
  p.k_per_split = pl.k_per_split;
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  int smode;
  if (p.group_size == 0 || p.group_size >= p.K) {
    smode = kPerChannel;
    p.group_size = 0;
  } else if (p.group_size % 32 == 0) {
    smode = kGroup32;
  } else if (p.group_size % 8 == 0) {
    smode = kGroup8;
  } else {
    smode = kGeneric;
  }
  const dim3 grid((unsigned)(pl.tiles_m * pl.tiles_n), 1, (unsigned)pl.split);
  hipError_t e;
  if (pl.cfg == 0) e = launch_cfg<64, 32>(p, grid, order, smode, qa4, s);
  else e = launch_cfg<128, 64>(p, grid, order, smode, qa4, s);
  if (e != hipSuccess || pl.split == 1) return e;
  const int64_t total = p.M * p.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, p.partial, p.bias, p.out, p.ldo, p.M, p.N, p.split);
  return hipGetLastError();
}

}  // namespace q4
