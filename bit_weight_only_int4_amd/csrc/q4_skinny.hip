// q4_skinny.hip -- MFMA GEMM for few activation rows (1 <= M <= 32) on
// gfx950: binary16 operands, fp32 accumulation, the arithmetic of the tiled
// prefill GEMM (q4_gemm.hip):
//
//   out[m, n] = sum_k RN16(x[m, k]) * RN16((q[n, k] - 8) * RN16(s[g(k), n]))
//               (+ bias[n]), summed in fp32 by the matrix unit.
//
// (page 1, stack entry #20752: binary16 multiplies into an fp32
// accumulator; page 1, stack entry #20798: every packed word crosses into
// the chip once and is unpacked once.)
//
// With few rows the tiled GEMM's 128-row tiles are mostly padding and its
// three launches (activation pre-pass, GEMM, split-K reduce) cost more than
// the weights take to stream.  Here one launch does the whole layer for the
// shapes it takes:
//  * The activations of the workgroup's K range are converted to binary16
//    (RN16) inside the kernel, once per workgroup, and stay in LDS for the
//    rest of it, in the operand order of the matrix instruction (below).
//    Only the M real rows are stored; the padding rows of a 16-row block
//    are zeros that never leave registers.
//  * Workgroups are persistent: each loops over blocks of output columns.
//    A wave streams the packed weights of its 32 columns (two 16-column
//    MFMA blocks) straight from HBM into registers with 16-byte loads, a
//    ring of D steps deep, and unpacks every word once into B operands.
//  * The eight waves of a workgroup split its column block along K when the
//    columns are few (narrow N) and add their partial sums through LDS in a
//    fixed order; with many columns every wave owns a column block and
//    stores it directly.  Only when the activations of one row block exceed
//    LDS is K also split across workgroups (grid.y), with fp32 partials in
//    the workspace and the shared split-K reduce.
//
// v_mfma_f32_16x16x32_f16 operand layout (wave64): lane l supplies A row
// l % 16 and B column l % 16, each with k-chunk l / 16 (8 binary16 values);
// D holds row 4 (l / 16) + v, column l % 16 in element v.  Any permutation
// of k that A and B share leaves the sum unchanged, so each lane's 16-byte
// weight load (32 consecutive k of its column, four packed words) feeds four
// MFMAs: MFMA t takes word t of every lane, i.e. k-chunk 4 g + t of the
// 128-k step for lane group g.  The activations are laid out in LDS so that
// lane (row m, group g) finds the matching eight values of MFMA t in one
// 16-byte slot, permuted inside the chunk like the nibbles of the word
// (pairs (i, i + 4)).
//
// Pages cited by number (the texts this layer is written from):
//   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
//           (its stack entries #20730 ... #20801);
//   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
//           (its stack entries #20917 ... #21005).
#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int SK_W = 8;       // waves per workgroup
constexpr int SK_STEP = 128;  // k per wave step (4 lane groups x 32 k)
constexpr int SK_D = 2;       // wave steps in a wave's load ring

// s_waitcnt vmcnt(N), other counters left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T>
__device__ __forceinline__ T* sk_uniform(T* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// One wave step's loads: for each of the two 16-column blocks, the lane's
// 16 packed bytes, its scale and (HASB) its column's bias.
struct SkSlot {
  uint32_t q[2][4];
  float s[2];
  float b[2];
};

template <bool S16>
__device__ __forceinline__ float sk_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (S16)
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// MB: 16-row MFMA blocks (1: M <= 16, 2: M <= 32).
template <int ORDER, bool PERCH, bool S16, bool HASB, int MB>
__global__ void __launch_bounds__(64 * SK_W)
gemm_skinny_kernel(const GemmParams p, const SkinnyPlan pl) {
  constexpr uint32_t SB = S16 ? 2 : 4;
  extern __shared__ __attribute__((aligned(16))) uint32_t sk_smem[];
  char* xs = reinterpret_cast<char*>(sk_smem);  // binary16 activations
  float* red = reinterpret_cast<float*>(xs + pl.x_lds);  // partial sums (wk > 1)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wkc = pl.wk;                 // waves along K
  const int wn = wave / wkc, wk = wave - wn * wkc;
  const int li = lane & 15, g = lane >> 4;
  const int M = (int)p.M;
  const int64_t N = p.N, K = p.K;
  const int z = blockIdx.y;
  const int64_t kz0 = (int64_t)z * pl.k_slice;
  const int64_t kz1 = kz0 + pl.k_slice < K ? kz0 + pl.k_slice : K;
  const int sps = (int)((kz1 - kz0 + SK_STEP - 1) / SK_STEP);  // steps in this slice
  const int spw = pl.spw;                // steps per wave and column block
  const int Gx = (int)gridDim.x;
  const int L = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  const int nblk = (int)((pl.blocks - L + Gx - 1) / Gx);  // column blocks of this workgroup
  const int T = nblk * spw;

  const int64_t Kp = (K + 1) >> 1;
  const __amdgpu_buffer_rsrc_t rq =
      sk_rsrc(p.qw, (uint64_t)(N - 1) * (uint64_t)p.ldq + (uint64_t)Kp);
  const void* sbase = S16 ? (const void*)p.scales16 : (const void*)p.scales;
  const __amdgpu_buffer_rsrc_t rs =
      sk_rsrc(sbase, PERCH ? (uint64_t)N * SB : ((uint64_t)(p.G - 1) * p.lds + (uint64_t)N) * SB);
  const __amdgpu_buffer_rsrc_t rb = sk_rsrc(p.bias, HASB ? (uint64_t)N * 4 : 0);
  // Steps past the workgroup's last one, and steps past the slice, issue the
  // same loads aimed at lines of the first activation row (resident in L2),
  // so that every step issues the same instructions and the ring's registers
  // stay put; they are never computed.
  const __amdgpu_buffer_rsrc_t rx =
      sk_rsrc(sk_uniform(p.x), (uint64_t)K * 4);
  const uint32_t xspan = (uint32_t)(K * 4) & ~1023u;
  const uint32_t dlane = ((uint32_t)(wave * 1024 + 16 * lane)) % (xspan ? xspan : 1024u);

  const uint32_t qg = 16u * (uint32_t)g;          // byte of the lane's chunk in a step
  const uint32_t kq0 = (uint32_t)(kz0 >> 1);      // first byte of the slice in a row
  const int l2g = p.log2_gs;
  auto issue = [&](int i, int sw, SkSlot& sl) {
    const int sidx = wk * spw + sw;
    const bool blive = i < nblk;  // a column block of this workgroup
    const bool live = blive && sidx < sps;
    const int64_t nb = ((int64_t)(L + i * Gx) * pl.wn + wn) * 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t n = nb + 16 * u + li;
      const uint32_t nc = (uint32_t)(n < N ? n : N - 1);
      const uint32_t qoff = live ? nc * (uint32_t)p.ldq + kq0 + 64u * (uint32_t)sidx + qg : dlane;
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(live ? rq : rx, qoff, 0, 2));
      sl.q[u][0] = v.x; sl.q[u][1] = v.y; sl.q[u][2] = v.z; sl.q[u][3] = v.w;
      uint32_t soff;
      if (PERCH) {
        soff = nc * SB;
      } else {
        const uint32_t grp = (uint32_t)((kz0 + SK_STEP * sidx + 32 * g) >> l2g);
        soff = (grp * (uint32_t)p.lds + nc) * SB;
      }
      sl.s[u] = sk_scale<S16>(live ? rs : rx, live ? soff : dlane);
      // the bias of every live block, also on a wave whose steps lie past
      // the slice: with waves split along K that wave still adds the bias
      // for its share of the block's sums
      if (HASB)
        sl.b[u] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(blive ? rb : rx, blive ? nc * 4u : dlane, 0, 0));
    }
  };

  // 1. The activations of the slice, RN16, into LDS.  16-byte slot of
  //    (step s, MFMA t, lane group g, row m): ((s * 4 + t) * 4 + g) * M + m;
  //    it holds k = kz0 + 128 s + 32 g + 8 t + (0..7) in nibble order, zeros
  //    past K.  A thread converts four 8-k chunks per round, their loads
  //    issued together (no branch around them: a chunk past K or past the
  //    last one reads the row start and is zeroed, or repeats the last chunk).  The ring's
  //    first D steps go out between the last round's loads and their use, so
  //    that the two latencies overlap.
  const int cpr = sps * 16;  // 8-k chunks per row
  const int total = M * cpr;
  const __amdgpu_buffer_rsrc_t rxa =
      sk_rsrc(sk_uniform(p.x), ((uint64_t)(M - 1) * (uint64_t)p.ldx + (uint64_t)K) * 4);
  constexpr int NT = 64 * SK_W;
  struct Stage {
    f4 v[4][2];
    int m[4], k[4];
  };
  auto stage_load = [&](int c0, Stage& st) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * NT < total ? c0 + u * NT : total - 1;
      st.m[u] = c / cpr;
      st.k[u] = c - st.m[u] * cpr;
      const int64_t k = kz0 + 8 * st.k[u];
      const uint32_t off = (uint32_t)(((int64_t)st.m[u] * p.ldx + (k < K ? k : 0)) * 4);
      st.v[u][0] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rxa, off, 0, 0));
      st.v[u][1] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rxa, off + 16, 0, 0));
    }
  };
  auto stage_store = [&](const Stage& st) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = kz0 + 8 * st.k[u] < K;
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = in ? st.v[u][0][e] : 0.0f;
        f[4 + e] = in ? st.v[u][1][e] : 0.0f;
      }
      h8 h;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) h[sl] = (_Float16)f[pair_k<ORDER>(sl >> 1, sl & 1)];
      const int s = st.k[u] >> 4, gg = (st.k[u] >> 2) & 3, t = st.k[u] & 3;
      // (a chunk past the last one repeats the last one: the same bytes to
      // the same slot)
      *reinterpret_cast<h8*>(xs + (((s * 4 + t) * 4 + gg) * M + st.m[u]) * 16) = h;
    }
  };
  const int rounds = (total + 4 * NT - 1) / (4 * NT);
  int c0 = (int)threadIdx.x;
  for (int r = 0; r + 1 < rounds; ++r, c0 += 4 * NT) {
    Stage st;
    stage_load(c0, st);
    __builtin_amdgcn_sched_barrier(0);
    stage_store(st);
  }
  Stage st;
  stage_load(c0, st);
  __builtin_amdgcn_sched_barrier(0);

  SkSlot ring[SK_D];
  int ii = 0, is = 0;  // issue position: column block, wave step
#pragma unroll
  for (int j = 0; j < SK_D; ++j) {
    issue(ii, is, ring[j]);
    if (++is == spw) { is = 0; ++ii; }
    __builtin_amdgcn_sched_barrier(0);
  }
  stage_store(st);
  __syncthreads();

  const Magic mg = Magic::make();
  f4 acc[2][MB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[u][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  bool mok[MB];
  int aoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    mok[mb] = li + 16 * mb < M;
    aoff[mb] = (g * M + li + 16 * mb) * 16;
  }
  const int tstride = 4 * M * 16;  // bytes between the MFMA slots of one step

  auto compute = [&](const SkSlot& sl, int sidx) {
    const char* ab = xs + sidx * 4 * tstride;
    // words of chunks past K (the last step of a K that is not a multiple
    // of 128) become 0x88888888: c = 0, so nothing past K enters the sum
    const bool pastk = kz0 + SK_STEP * sidx + 32 * g >= K;
    h2 s16[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) s16[u] = splat_f16(sl.s[u]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        a[mb] = h8{0, 0, 0, 0, 0, 0, 0, 0};
        if (mok[mb]) a[mb] = *reinterpret_cast<const h8*>(ab + t * tstride + aoff[mb]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t w = pastk ? 0x88888888u : sl.q[u][t];
        h2 c[4];
        unpack_word(w, mg, c);
        h2 d[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) d[pp] = dequant_pair_f16(c[pp], s16[u]);
        const h8 b = h8{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[u][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], b, acc[u][mb], 0, 0, 0);
      }
    }
  };

  // out[m, n] (+ bias) or the slice's partial, for element v of block (u, mb)
  float* const dst = pl.split > 1 ? p.partial + (int64_t)z * M * N : p.out;
  const int64_t dpitch = pl.split > 1 ? N : p.ldo;
  const bool addb = HASB && pl.split == 1;
  auto store = [&](int64_t nb, int u, int mb, int v, float val, float bias) {
    const int m = 16 * mb + 4 * g + v;
    const int64_t n = nb + 16 * u + li;
    if (m < M && n < N) dst[(int64_t)m * dpitch + n] = addb ? val + bias : val;
  };

  // A column block leaves once its last step is in.  With waves split along
  // K, each wave parks its sums in LDS; then wave wk of the column group
  // adds, for its share of the elements, the wkc partials in wave order.
  auto finish = [&](int i, const float (&bias)[2]) {
    const int64_t nb = ((int64_t)(L + i * Gx) * pl.wn + wn) * 32;
    if (wkc == 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) store(nb, u, mb, v, acc[u][mb][v], bias[u]);
    } else {
      constexpr int NV = 2 * MB * 4;  // sums per lane
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(wave * NV + (u * MB + mb) * 4 + v) * 64 + lane] = acc[u][mb][v];
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int idx = (u * MB + mb) * 4 + v;
            if (idx % wkc == wk) {
              float sum = 0.0f;
              for (int j = 0; j < wkc; ++j) sum += red[((wn * wkc + j) * NV + idx) * 64 + lane];
              store(nb, u, mb, v, sum, bias[u]);
            }
          }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[u][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // 2. whole rounds of D steps; every step issues the loads of the step D
  //    later (the same instructions on every path), computes if it is one of
  //    the workgroup's steps inside the slice, and closes its column block
  //    after its last step.  T and the block ends are the same for every
  //    wave of the workgroup, so the barriers of finish() pair up.
  int ci = 0, cs = 0;  // compute position
  const int TR = (T + SK_D - 1) / SK_D * SK_D;
  for (int t0 = 0; t0 < TR; t0 += SK_D) {
#pragma unroll
    for (int j = 0; j < SK_D; ++j) {
      const bool run = t0 + j < T;
      const int sidx = wk * spw + cs;
      if (run && sidx < sps) compute(ring[j], sidx);
      float bias[2] = {0.0f, 0.0f};
      if (HASB) { bias[0] = ring[j].b[0]; bias[1] = ring[j].b[1]; }
      const bool last = run && cs == spw - 1;
      const int cblk = ci;
      __builtin_amdgcn_sched_barrier(0);
      issue(ii, is, ring[j]);
      if (++is == spw) { is = 0; ++ii; }
      __builtin_amdgcn_sched_barrier(0);
      if (run && ++cs == spw) { cs = 0; ++ci; }
      if (last) finish(cblk, bias);
    }
  }
  // the ring's last loads (past the end) are drained before the wave exits
  sk_wait_vmcnt<0>();
}

template <int ORDER, bool PERCH, bool S16, bool HASB, int MB>
hipError_t launch_sk(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  auto kern = gemm_skinny_kernel<ORDER, PERCH, S16, HASB, MB>;
  const size_t lds = (size_t)pl.x_lds + (size_t)pl.red_lds;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.grid, (unsigned)pl.split), dim3(64 * SK_W), lds, s,
                     p, pl);
  return hipGetLastError();
}

template <int ORDER, bool PERCH, bool S16>
hipError_t launch_sk_b(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  const bool hasb = p.bias != nullptr;
  if (pl.mb == 1)
    return hasb ? launch_sk<ORDER, PERCH, S16, true, 1>(p, pl, s)
                : launch_sk<ORDER, PERCH, S16, false, 1>(p, pl, s);
  return hasb ? launch_sk<ORDER, PERCH, S16, true, 2>(p, pl, s)
              : launch_sk<ORDER, PERCH, S16, false, 2>(p, pl, s);
}

template <int ORDER>
hipError_t launch_sk_o(const GemmParams& p, const SkinnyPlan& pl, bool perch, hipStream_t s) {
  const bool s16 = p.scales16 != nullptr;
  if (perch)
    return s16 ? launch_sk_b<ORDER, true, true>(p, pl, s) : launch_sk_b<ORDER, true, false>(p, pl, s);
  return s16 ? launch_sk_b<ORDER, false, true>(p, pl, s) : launch_sk_b<ORDER, false, false>(p, pl, s);
}

}  // namespace

// LDS for the activations of one slice (M rows x k_slice binary16) plus,
// with waves split along K, the partial sums (8 waves x 8 or 16 floats per
// lane).  One row of the plan per call, from the sizes alone.
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  SkinnyPlan pl{};
  const bool perch = group_size == 0 || group_size >= K;
  const bool pow2 = group_size >= 32 && (group_size & (group_size - 1)) == 0;
  pl.ok = M >= 1 && M <= 32 && N >= 1 && K >= SK_STEP && K % 32 == 0 && (perch || pow2) &&
          K <= ((int64_t)1 << 24);
  if (!pl.ok) return pl;
  pl.mb = M <= 16 ? 1 : 2;
  const int64_t red = (int64_t)SK_W * 2 * pl.mb * 4 * 64 * 4;  // bytes
  constexpr int64_t kLds = 160 * 1024;
  const int64_t steps = (K + SK_STEP - 1) / SK_STEP;
  const int64_t per_step = (int64_t)SK_STEP * M * 2;
  const int64_t max_steps = (kLds - red) / per_step;
  int64_t split = (steps + max_steps - 1) / max_steps;
  const int64_t sps = (steps + split - 1) / split;
  split = (steps + sps - 1) / sps;
  pl.split = (int)split;
  pl.k_slice = sps * SK_STEP;
  // waves along K: as few as leave at least 256 workgroup column blocks
  const int64_t nb32 = (N + 31) / 32;
  int wk = 8;
  for (int c = 1; c <= 8; c *= 2)
    if ((nb32 * c + 7) / 8 >= 256) { wk = c; break; }
  while (wk > 1 && wk > sps) wk /= 2;
  pl.wk = wk;
  pl.wn = SK_W / wk;
  pl.spw = (int)((sps + wk - 1) / wk);
  pl.blocks = (nb32 + pl.wn - 1) / pl.wn;
  pl.x_lds = (int)(sps * per_step);
  pl.red_lds = wk > 1 ? (int)red : 0;
  const int64_t lds = pl.x_lds + pl.red_lds;
  const int64_t occ = lds * 2 <= kLds ? 2 : 1;  // workgroups per CU
  int64_t grid = 256 * occ / split;
  if (grid < 1) grid = 1;
  if (grid > pl.blocks) grid = pl.blocks;
  pl.grid = (int)grid;
  return pl;
}

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  const SkinnyPlan pl = plan_skinny(M, N, K, group_size);
  if (!pl.ok || pl.split == 1) return 0;
  return (size_t)pl.split * (size_t)M * (size_t)N * sizeof(float);
}

// Pointer-dependent conditions of the skinny kernel: dword-aligned weight
// rows (16-byte loads) and every byte offset of its buffer loads below 2^32.
bool skinny_fits(const GemmParams& p, const SkinnyPlan& pl, bool qa4) {
  if (!pl.ok || !qa4) return false;
  const uint64_t qbytes = (uint64_t)p.N * (uint64_t)p.ldq;
  const uint64_t sb = p.scales16 ? 2 : 4;
  const uint64_t sbytes = ((uint64_t)p.G * (uint64_t)p.lds + (uint64_t)p.N) * sb;
  const uint64_t xbytes = ((uint64_t)(p.M - 1) * (uint64_t)p.ldx + (uint64_t)p.K) * 4;
  return qbytes < (1ull << 32) - 64 && sbytes < (1ull << 32) && xbytes < (1ull << 32);
}

hipError_t launch_skinny(const GemmParams& p0, const SkinnyPlan& pl, int order, void* workspace,
                         hipStream_t s) {
  GemmParams p = p0;
  const bool perch = p.group_size == 0 || p.group_size >= p.K;
  p.log2_gs = -1;
  if (!perch) {
    int l2 = 0;
    while ((1LL << l2) < p.group_size) ++l2;
    p.log2_gs = l2;
  }
  p.partial = reinterpret_cast<float*>(workspace);
  const hipError_t e = order == 0 ? launch_sk_o<0>(p, pl, perch, s) : launch_sk_o<1>(p, pl, perch, s);
  if (e != hipSuccess || pl.split == 1) return e;
  return launch_splitk_reduce(p.partial, p.bias, p.out, p.ldo, p.M, p.N, pl.split, s);
}

}  // namespace q4
