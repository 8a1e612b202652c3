// q4_bwd_mfma.hip -- the input gradient on MFMA (Q4_MATH_F16), for gfx950.
//
//   d_x[m, k] = sum_n RN16(d_out[m, n]) * RN16((q[n, k] - 8) * RN16(s[g(k), n])),
//               summed in fp32
//
// the contraction over N of page 3, "Add fp32 matmul ops (mm, bmm, linear)",
// stack entry #20943, with the operands the forward's binary16 path feeds to
// MFMA (page 1, stack entry #20752: binary16 multiply, fp32 accumulator).
//
// The packed weight is stored along K ([N, K/2]) while this contraction runs
// along N, so each weight tile is dequantized once into LDS transposed,
// [k][n], where an MFMA B fragment (8 consecutive n of one column k) is one
// 16-byte read:
//  * A pre-pass rounds d_out to binary16 once, zero-padded to whole tiles.
//  * Workgroups own 128 (m) x 128 (k) output tiles and step through N 64 at
//    a time.  Each of the 4 waves owns 32 columns k and all 128 rows: four
//    v_mfma_f32_32x32x16_f16 blocks share one B fragment.
//  * Thread t stages the packed words of rows n = 2 (t % 16) + 32 h and
//    n + 1 (h = 0, 1) at the 8 k of word t / 16, unpacks them (q4_device.h),
//    applies each row's scale as RN16(c * RN16(s)) and writes the 8 (n, n + 1)
//    pairs of binary16 weights as dwords.  Each packed word is read and
//    unpacked once per output tile.
//  * Double-buffered LDS with the next step's global loads in registers
//    while the current step's MFMAs run; one barrier per step.
//  * Deep N on few tiles is split over grid.z; fp32 partials go to the
//    workspace and the split-K reduce kernel adds them in split order, so
//    results are deterministic.
// One group per packed word: group_size a multiple of 8, or per-channel.
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

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BB_M = 128;     // rows m per tile
constexpr int BB_K = 128;     // output columns k per tile
constexpr int BB_S = 64;      // contraction step over n (32 or 64; 64 measured
                              // faster from 512 rows on)
constexpr int BB_NT = 256;
// row pitch, in floats, of the output tile the epilogue stages in LDS (the
// two row halves of one LDS store land on disjoint banks)
constexpr int BB_EPI_TP = 136;
// LDS row pitch in halves: NS + 8 (80 or 144 bytes), so the 16 rows that
// one 16-lane group of a ds_read_b128 reads fall on 16 distinct 4-bank
// groups
template <int NS>
constexpr int bb_pitch() { return NS + 8; }

// d16[r][n] = RN16(d_out[r][n]) for r < M, n < N, else 0; [mp][np].  A
// workgroup covers 2048 n of a row; grid.y strides the rows.
__global__ void __launch_bounds__(256)
dout16_kernel(const float* __restrict__ d, int64_t ldd, int64_t M, int64_t N,
              _Float16* __restrict__ d16, int64_t mp, int64_t np) {
  const int64_t n0 = (int64_t)blockIdx.x * 2048 + 8 * threadIdx.x;
  if (n0 >= np) return;
  for (int64_t r = blockIdx.y; r < mp; r += gridDim.y) {
    const float* src = d + r * ldd + n0;
    h8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)((r < M && n0 + i < N) ? src[i] : 0.0f);
    *reinterpret_cast<h8*>(d16 + r * np + n0) = h;
  }
}

template <int ORDER, bool QA4, int NS>
__global__ void __launch_bounds__(BB_NT)
bwd_mfma_kernel(const BwdMfmaParams p) {
  constexpr int PITCH = bb_pitch<NS>();
  constexpr int AP = NS / 16;  // 16-byte d_out pieces per thread per step
  constexpr int BP = NS / 32;  // row pairs per thread per step
  struct Smem {
    _Float16 a[2][BB_M * PITCH];
    _Float16 b[2][BB_K * PITCH];
  };
  static_assert(sizeof(Smem) >= BB_M * BB_EPI_TP * sizeof(float),
                "the epilogue stages the output tile in the operand buffers");
  __shared__ __attribute__((aligned(16))) Smem sm;
  auto& As = sm.a;
  auto& Bs = sm.b;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, lb = lane >> 5;
  const uint32_t tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(tile % (uint32_t)p.tiles_m) * BB_M;
  const int64_t k0 = (int64_t)(tile / (uint32_t)p.tiles_m) * BB_K;
  const int z = blockIdx.z;
  const int64_t nz0 = (int64_t)z * p.n_per_split;
  const int64_t nz1 = (nz0 + p.n_per_split < p.N) ? nz0 + p.n_per_split : p.N;
  const int nsteps = (int)((nz1 - nz0 + NS - 1) / NS);

  // this thread's weight word: rows 2 (pp + 16 h) and 2 (pp + 16 h) + 1 of
  // each step (h < BP), k kw .. kw + 7 (one group)
  const int pp = tid & 15, wd = tid >> 4;
  const int64_t kw = k0 + 8 * wd;
  const int64_t row_bytes = (p.K + 1) >> 1;
  const bool kin = kw < p.K, kfull = kw + 8 <= p.K;
  int64_t g = 0;
  if (p.group_size > 0 && kin) g = p.log2_gs >= 0 ? (kw >> p.log2_gs) : kw / p.group_size;
  const float* srow = p.scales + g * p.lds;

  struct Stage {
    u32x4 a[AP];         // 16-byte pieces of the binary16 d_out tile
    uint32_t q[2 * BP];  // packed words of rows 2 (pp + 16 h) + e
    float s[2 * BP];     // their scales
  };

  auto load = [&](int step, Stage& st) {
    const int64_t nb = nz0 + (int64_t)step * NS;
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const int u = tid + BB_NT * j;  // row u / (NS / 8), piece u % (NS / 8)
      st.a[j] = *reinterpret_cast<const u32x4*>(p.d16 + (m0 + u / (NS / 8)) * p.d16_pitch +
                                                 nb + 8 * (u % (NS / 8)));
    }
#pragma unroll
    for (int h = 0; h < 2 * BP; ++h) {
      const int64_t n = nb + 2 * (pp + 16 * (h >> 1)) + (h & 1);
      uint32_t v = 0x88888888u;  // code 8 = weight 0
      float sc = 0.0f;
      if (n < nz1 && kin) {
        const uint8_t* row = p.qw + n * p.ldq + (kw >> 1);
        if (QA4 && kfull) {
          v = *reinterpret_cast<const uint32_t*>(row);
        } else {
          v = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            v |= ((kw >> 1) + b < row_bytes ? (uint32_t)row[b] : 0x88u) << (8 * b);
        }
        sc = srow[n];
      }
      st.q[h] = v;
      st.s[h] = sc;
    }
  };

  const Magic mg = Magic::make();
  auto store = [&](const Stage& st, _Float16* as, _Float16* bs) {
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const int u = tid + BB_NT * j;
      *reinterpret_cast<u32x4*>(as + (u / (NS / 8)) * PITCH + 8 * (u % (NS / 8))) = st.a[j];
    }
#pragma unroll
    for (int h = 0; h < BP; ++h) {
      h2 ca[4], cb[4];
      unpack_word(st.q[2 * h], mg, ca);
      unpack_word(st.q[2 * h + 1], mg, cb);
      const h2 sa = splat_f16(st.s[2 * h]), sb = splat_f16(st.s[2 * h + 1]);
      h2 da[4], db[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        da[i] = dequant_pair_f16(ca[i], sa);
        db[i] = dequant_pair_f16(cb[i], sb);
      }
      // k offset j of the word sits in nibble nibble_k(j) (an involution),
      // which unpack_word put in pair (nibble & 3), half (nibble >> 2)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = nibble_k<ORDER>(j);
        const _Float16 va = (i >> 2) ? da[i & 3].y : da[i & 3].x;
        const _Float16 vb = (i >> 2) ? db[i & 3].y : db[i & 3].x;
        *reinterpret_cast<h2*>(bs + (8 * wd + j) * PITCH + 2 * (pp + 16 * h)) = h2{va, vb};
      }
    }
  };

  f16v acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // B fragment: column k = 32 w + li, n = 16 t + 8 lb .. + 7; A fragment:
  // row 32 i + li, the same n
  auto compute = [&](const _Float16* as, const _Float16* bs) {
#pragma unroll
    for (int t = 0; t < NS / 16; ++t) {
      const h8 b = *reinterpret_cast<const h8*>(bs + (32 * w + li) * PITCH + 16 * t + 8 * lb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h8 a = *reinterpret_cast<const h8*>(as + (32 * i + li) * PITCH + 16 * t + 8 * lb);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
      }
    }
  };

  // Step s's MFMAs run on LDS buffer s & 1 while the loads of step s + 1
  // are in flight; step s + 1 is then written to the other buffer.  One
  // barrier per step: a buffer is rewritten only after every wave has passed
  // the barrier that ended the step reading it.  (Deeper register rings
  // measured slower: they cost occupancy.)
  Stage st;
  if (nsteps > 0) {
    load(0, st);
    store(st, As[0], Bs[0]);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load(s + 1, st);
    compute(As[buf], Bs[buf]);
    if (s + 1 < nsteps) store(st, As[buf ^ 1], Bs[buf ^ 1]);
    __syncthreads();
  }

  // Epilogue (the loop's last barrier has freed the operand buffers): the
  // tile goes through LDS and leaves as 16-byte row-contiguous stores,
  // non-temporal for d_x.  Lane l, element v of a 32x32 block holds row
  // 8 * (v / 4) + 4 * (l / 32) + v % 4 and column l % 32.
  float* ctile = reinterpret_cast<float*>(&sm);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      ctile[(32 * i + 8 * (v >> 2) + 4 * lb + (v & 3)) * BB_EPI_TP + 32 * w + li] = acc[i][v];
  __syncthreads();
  const int c4 = tid & 31;  // column quad of the tile
  const int64_t col = k0 + 4 * c4;
  float* dst0;
  int64_t pitch;
  bool vec;
  if (p.split > 1) {
    dst0 = p.partial + (int64_t)z * p.M * p.K;
    pitch = p.K;
    vec = p.K % 4 == 0 && reinterpret_cast<uintptr_t>(dst0) % 16 == 0;
  } else {
    dst0 = p.dx;
    pitch = p.lddx;
    vec = p.lddx % 4 == 0 && reinterpret_cast<uintptr_t>(p.dx) % 16 == 0;
  }
#pragma unroll 4
  for (int j = 0; j < BB_M / 8; ++j) {
    const int r = (tid >> 5) + 8 * j;
    const int64_t row = m0 + r;
    if (row >= p.M) break;
    const f4 v = *reinterpret_cast<const f4*>(ctile + r * BB_EPI_TP + 4 * c4);
    float* dst = dst0 + row * pitch + col;
    if (vec && col + 4 <= p.K) {
      if (p.split > 1)
        *reinterpret_cast<f4*>(dst) = v;
      else
        __builtin_nontemporal_store(v, reinterpret_cast<f4*>(dst));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < p.K) dst[e] = v[e];
    }
  }
}

template <int ORDER>
hipError_t launch_bwd_mfma_t(const BwdMfmaParams& p, dim3 grid, bool qa4, hipStream_t s) {
  if (qa4)
    hipLaunchKernelGGL((bwd_mfma_kernel<ORDER, true, BB_S>), grid, dim3(BB_NT), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_mfma_kernel<ORDER, false, BB_S>), grid, dim3(BB_NT), 0, s, p);
  return hipGetLastError();
}

constexpr size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

BwdMfmaPlan plan_bwd_mfma(int64_t M, int64_t N, int64_t K) {
  BwdMfmaPlan pl{};
  pl.tiles_m = (M + BB_M - 1) / BB_M;
  pl.tiles_k = (K + BB_K - 1) / BB_K;
  pl.mp = pl.tiles_m * BB_M;
  const int64_t steps = (N + BB_S - 1) / BB_S;
  pl.np = steps * BB_S;
  // split N while the tiles alone leave CUs without 2 workgroups (the LDS
  // holds two) and each split keeps at least 4 steps (measured best of
  // several such rules over M = 16 .. 2048)
  const int64_t tiles = pl.tiles_m * pl.tiles_k;
  int64_t split = 1;
  while (tiles * split * 2 <= 512 && steps / (split * 2) >= 4) split *= 2;
  const int64_t per = (steps + split - 1) / split;
  pl.n_per_split = per * BB_S;
  pl.split = (int)((N + pl.n_per_split - 1) / pl.n_per_split);
  return pl;
}

size_t bwd_mfma_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const BwdMfmaPlan pl = plan_bwd_mfma(M, N, K);
  size_t b = align256((size_t)pl.mp * (size_t)pl.np * 2);
  if (pl.split > 1) b += (size_t)pl.split * (size_t)M * (size_t)K * sizeof(float);
  return b;
}

hipError_t launch_bwd_mfma(const BwdParams& q, int order, bool qa4, void* workspace,
                           hipStream_t s) {
  const BwdMfmaPlan pl = plan_bwd_mfma(q.M, q.N, q.K);
  BwdMfmaParams p{};
  p.d16 = reinterpret_cast<_Float16*>(workspace);
  p.d16_pitch = pl.np;
  p.qw = q.qw;
  p.ldq = q.ldq;
  p.scales = q.scales;
  p.lds = q.lds;
  p.group_size = q.group_size >= q.K ? 0 : q.group_size;  // one group: per-channel
  p.log2_gs = -1;
  if (p.group_size > 0 && (p.group_size & (p.group_size - 1)) == 0) {
    int l2 = 0;
    while ((1LL << l2) < p.group_size) ++l2;
    p.log2_gs = l2;
  }
  p.dx = q.dx;
  p.lddx = q.lddx;
  p.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                       align256((size_t)pl.mp * (size_t)pl.np * 2));
  p.M = q.M;
  p.N = q.N;
  p.K = q.K;
  p.n_per_split = pl.n_per_split;
  p.split = pl.split;
  p.tiles_m = (int32_t)pl.tiles_m;
  p.tiles_k = (int32_t)pl.tiles_k;
  // 1. d_out to binary16
  const dim3 dgrid((unsigned)((pl.np + 2047) / 2048), (unsigned)(pl.mp < 65535 ? pl.mp : 65535));
  hipLaunchKernelGGL(dout16_kernel, dgrid, dim3(256), 0, s, q.dout, q.lddo, q.M, q.N,
                     reinterpret_cast<_Float16*>(workspace), pl.mp, pl.np);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. the GEMM
  const dim3 grid((unsigned)(pl.tiles_m * pl.tiles_k), 1, (unsigned)pl.split);
  e = order == 0 ? launch_bwd_mfma_t<0>(p, grid, qa4, s) : launch_bwd_mfma_t<1>(p, grid, qa4, s);
  if (e != hipSuccess || pl.split == 1) return e;
  // 3. the split partials, in split order
  return launch_splitk_reduce(p.partial, nullptr, q.dx, q.lddx, q.M, q.K, pl.split, s);
}

}  // namespace q4
