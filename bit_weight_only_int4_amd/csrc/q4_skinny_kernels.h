// q4_skinny_kernels.h -- MFMA GEMM for few activation rows (1 <= M <= 1024) on
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
//    read the last real row, and their outputs are never stored.
//  * Workgroups are persistent: each loops over blocks of output columns.
//    A wave streams the packed weights of its 32 columns (two 16-column
//    MFMA blocks) straight from HBM into registers with 16-byte loads, a
//    ring of D steps deep, and unpacks every word once into B operands.
//  * More than 32 rows go in row blocks of 32, each its own set of
//    workgroups; neighbouring workgroups (one XCD) take the same columns for
//    different row blocks, so the second read of the weights meets the
//    first in that XCD's L2.
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
// The plan and the choice of kernel are in q4_skinny.hip; each nibble order
// is compiled in its own translation unit (q4_skinny_o0.hip,
// q4_skinny_o1.hip), which instantiates launch_skinny_kernels<ORDER>.  Not
// part of the public ABI.
//
// Pages cited by number (the texts this layer is written from):
//   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
//           (its stack entries #20730 ... #20801);
//   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
//           (its stack entries #20917 ... #21005).
#pragma once

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int SK_W = 8;       // waves per workgroup
constexpr int SK_STEP = 128;  // k per wave step (4 lane groups x 32 k)

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

// One wave step's loads: for each of the NI 16-column blocks, the lane's 16
// packed bytes, its scale and (HASB) its column's bias.
template <int NI>
struct SkSlot {
  uint32_t q[NI][4];
  float s[NI];
  float b[NI];
};

template <bool S16>
__device__ __forceinline__ float sk_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (S16)
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// How the scale meets the sum.  The operands stay binary16 and the sums
// fp32 in every mode; where one scale covers a whole 128-k step it is taken
// out of that step's sum (exact in real arithmetic), which spares the
// per-element multiply and its binary16 rounding of c * s:
//   SC_ELEM:    groups of 32 or 64: B = RN16(c * RN16(s)), the tiled GEMM's
//               operand;
//   SC_STEP:    power-of-two groups >= 128: B = c (exact), the step's MFMA
//               sum times s (one fp32 multiply-add into the accumulator);
//   SC_CHANNEL: per-channel scales: B = c, the whole sum times s at the end;
//   SC_ELEM_KT: SC_ELEM with K % 32 != 0 (K % 8 == 0): the 32-k chunk that
//               straddles K gets a zero scale for its 8-k words past K.
enum SkScale : int { SC_ELEM = 0, SC_STEP = 1, SC_CHANNEL = 2, SC_ELEM_KT = 3 };

// MB: 16-row MFMA blocks per row block (1: <= 16 rows, 2: <= 32).  NI: 16-column blocks
// per wave (2 or 4: 32 or 64 columns, NI 16-byte weight loads per lane and
// step, every A operand shared by NI MFMAs).
template <int ORDER, int SC, bool S16, bool HASB, int MB, int NI>
__global__ void __launch_bounds__(64 * SK_W)
gemm_skinny_kernel(const GemmParams p, const SkinnyPlan pl) {
  constexpr int D = 2;  // wave steps in a wave's load ring
  constexpr bool PERCH = SC == SC_CHANNEL;
  constexpr uint32_t SB = S16 ? 2 : 4;
  extern __shared__ __attribute__((aligned(16))) uint32_t sk_smem[];
  char* xs = reinterpret_cast<char*>(sk_smem);  // binary16 activations
  float* red = reinterpret_cast<float*>(xs + pl.x_lds);  // partial sums (wk > 1)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wkc = pl.wk;                 // waves along K
  const int wn = wave / wkc, wk = wave - wn * wkc;
  const int li = lane & 15, g = lane >> 4;
  // Row blocks of pl.mrows rows (grid of pl.mz of them): logical workgroup L
  // takes row block L % mz for good, and column blocks of the workgroups
  // L / mz; neighbouring logical ids (one XCD) share their column blocks,
  // so the weights they stream meet in that XCD's L2.
  const int Gx = (int)gridDim.x;
  const int Lall = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  const int zm = Lall % pl.mz;
  const int L = Lall / pl.mz;                // this workgroup's rank among Gb
  const int Gb = Gx / pl.mz;                 // workgroups per row block
  const int64_t mrow0 = (int64_t)zm * pl.mrows;
  const int M = (int)(p.M - mrow0 < pl.mrows ? p.M - mrow0 : pl.mrows);  // rows here
  const float* const xrows = p.x + mrow0 * p.ldx;
  const int64_t N = p.N, K = p.K;
  const int z = blockIdx.y;
  const int64_t kz0 = (int64_t)z * pl.k_slice;
  const int64_t kz1 = kz0 + pl.k_slice < K ? kz0 + pl.k_slice : K;
  const int sps = (int)((kz1 - kz0 + SK_STEP - 1) / SK_STEP);  // steps in this slice
  const int spw = pl.spw;                // steps per wave and column block
  const int nblk = (int)((pl.blocks - L + Gb - 1) / Gb);  // column blocks of this workgroup
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
      sk_rsrc(sk_uniform(xrows), (uint64_t)K * 4);
  const uint32_t xspan = (uint32_t)(K * 4) & ~1023u;
  const uint32_t dlane = ((uint32_t)(wave * 1024 + 16 * lane)) % (xspan ? xspan : 1024u);

  const uint32_t qg = 16u * (uint32_t)g;          // byte of the lane's chunk in a step
  const uint32_t kq0 = (uint32_t)(kz0 >> 1);      // first byte of the slice in a row
  const int l2g = p.log2_gs;
  auto issue = [&](int i, int sw, SkSlot<NI>& sl) {
    const int sidx = wk * spw + sw;
    const bool blive = i < nblk;  // a column block of this workgroup
    const bool live = blive && sidx < sps;
    const int64_t nb = ((int64_t)(L + i * Gb) * pl.wn + wn) * (16 * NI);
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int64_t n = nb + 16 * u + li;
      const uint32_t nc = (uint32_t)(n < N ? n : N - 1);
      const uint32_t qoff = live ? nc * (uint32_t)p.ldq + kq0 + 64u * (uint32_t)sidx + qg : dlane;
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(live ? rq : rx, qoff, 0, 2));
      sl.q[u][0] = v.x; sl.q[u][1] = v.y; sl.q[u][2] = v.z; sl.q[u][3] = v.w;
      // (a per-channel scale is applied at the block's end, by whichever
      // wave adds up the block: loaded for every live block, like the bias)
      if (PERCH) {
        sl.s[u] = sk_scale<S16>(blive ? rs : rx, blive ? nc * SB : dlane);
      } else {
        const uint32_t grp = (uint32_t)((kz0 + SK_STEP * sidx + 32 * g) >> l2g);
        sl.s[u] = sk_scale<S16>(live ? rs : rx, live ? (grp * (uint32_t)p.lds + nc) * SB : dlane);
      }
      // the bias of every live block, also on a wave whose steps lie past
      // the slice: with waves split along K that wave still adds the bias
      // for its share of the block's sums
      if (HASB)
        sl.b[u] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(blive ? rb : rx, blive ? nc * 4u : dlane, 0, 0));
    }
  };

  // 1. The activations of the slice, RN16, into LDS.  16-byte slot of row
  //    m, chunk c: m * cpr + (c ^ (m & 15)); it holds k = kz0 + 8 c + (0..7)
  //    in nibble order, zeros past K.  MFMA t of step s reads chunk
  //    16 s + 4 g + t for lane group g.  The XOR keeps a chunk inside its
  //    aligned group of 16 and spreads both a wave's staging stores
  //    (consecutive chunks of one row) and its operand reads (16 rows of one
  //    chunk per lane group) over 16 different groups of four banks; rows
  //    cpr slots apart without it (cpr a multiple of 16) put every store of a
  //    wave on the same four banks.  A thread converts four 8-k chunks per
  //    round, their loads issued together (no branch around them: a chunk
  //    past K or past the last one reads the row start and is zeroed, or
  //    repeats the last chunk).  The ring's first D steps go out between the
  //    last round's loads and their use, so that the two latencies overlap.
  const int cpr = sps * 16;  // 8-k chunks per row
  const int total = M * cpr;
  const __amdgpu_buffer_rsrc_t rxa =
      sk_rsrc(sk_uniform(xrows), ((uint64_t)(M - 1) * (uint64_t)p.ldx + (uint64_t)K) * 4);
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
      // (a chunk past the last one repeats the last one: the same bytes to
      // the same slot)
      *reinterpret_cast<h8*>(xs + (st.m[u] * cpr + (st.k[u] ^ (st.m[u] & 15))) * 16) = h;
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

  SkSlot<NI> ring[D];
  int ii = 0, is = 0;  // issue position: column block, wave step
#pragma unroll
  for (int j = 0; j < D; ++j) {
    issue(ii, is, ring[j]);
    if (++is == spw) { is = 0; ++ii; }
    __builtin_amdgcn_sched_barrier(0);
  }
  stage_store(st);
  __syncthreads();

  const Magic mg = Magic::make();
  f4 acc[NI][MB];
#pragma unroll
  for (int u = 0; u < NI; ++u)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[u][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // A operands: lane (row m, group g).  Rows m >= M read row M - 1: an
  // output row depends on its own A row only, and rows >= M are never stored.
  int aoff[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = li + 16 * mb < M ? li + 16 * mb : M - 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[mb][t] = (m * cpr + ((4 * g + t) ^ (m & 15))) * 16;
  }

  auto compute = [&](const SkSlot<NI>& sl, int sidx) {
    const char* ab = xs + sidx * 256;  // chunk 16 sidx of row 0
    h8 a[4][MB];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[t][mb] = *reinterpret_cast<const h8*>(ab + aoff[mb][t]);
    if constexpr (SC == SC_ELEM || SC == SC_ELEM_KT) {
      // chunks past K (the last step of a K that is not a multiple of 128)
      // get a zero scale, so that whatever bytes they read give w = 0; with
      // K % 32 != 0 so do the 8-k words past K of the chunk that straddles
      // it (bytes of the row pitch, of the next row, or zeros past the
      // array: a code times a zero scale is 0 whatever the code)
      const int64_t kc = kz0 + SK_STEP * sidx + 32 * g;  // the lane's chunk
      const bool pastk = kc >= K;
      h2 s16[NI];
#pragma unroll
      for (int u = 0; u < NI; ++u) s16[u] = splat_f16(pastk ? 0.0f : sl.s[u]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < NI; ++u) {
          h2 c[4];
          unpack_word(sl.q[u][t], mg, c);
          h2 su = s16[u];
          if constexpr (SC == SC_ELEM_KT) {
            if (kc + 8 * t >= K) su = h2{(_Float16)0.0f, (_Float16)0.0f};
          }
          h2 d[4];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) d[pp] = dequant_pair_f16(c[pp], su);
          const h8 bv = h8{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[u][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][mb], bv, acc[u][mb], 0, 0, 0);
        }
    } else {
      // B = c exactly: chunks past K, and with K % 32 != 0 the 8-k words
      // past K of the chunk that straddles it (bytes of the row pitch, of the
      // next row, or zeros past the array), meet activations staged as zero,
      // and c is finite, so they add exactly 0
      f4 st[NI][MB];
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          st[u][mb] = SC == SC_CHANNEL ? acc[u][mb] : f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < NI; ++u) {
          h2 c[4];
          unpack_word(sl.q[u][t], mg, c);
          const h8 bv = h8{c[0].x, c[0].y, c[1].x, c[1].y, c[2].x, c[2].y, c[3].x, c[3].y};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            st[u][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][mb], bv, st[u][mb], 0, 0, 0);
        }
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (SC == SC_CHANNEL) {
            acc[u][mb] = st[u][mb];
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[u][mb][v] = __builtin_fmaf(sl.s[u], st[u][mb][v], acc[u][mb][v]);
          }
        }
    }
  };

  // out[m, n] (+ bias) or the slice's partial, for element v of block (u, mb)
  const int64_t dpitch = pl.split > 1 ? N : p.ldo;
  float* const dst = (pl.split > 1 ? p.partial + (int64_t)z * p.M * N : p.out) + mrow0 * dpitch;
  const bool addb = HASB && pl.split == 1;
  auto store = [&](int64_t nb, int u, int mb, int v, float val, float scale, float bias) {
    const int m = 16 * mb + 4 * g + v;
    const int64_t n = nb + 16 * u + li;
    if (PERCH) val *= scale;
    if (m < M && n < N) dst[(int64_t)m * dpitch + n] = addb ? val + bias : val;
  };

  // A column block leaves once its last step is in.  With waves split along
  // K, each wave parks its sums in LDS; then wave wk of the column group
  // adds, for its share of the elements, the wkc partials in wave order.
  auto finish = [&](int i, const float (&scale)[NI], const float (&bias)[NI]) {
    const int64_t nb = ((int64_t)(L + i * Gb) * pl.wn + wn) * (16 * NI);
    if (wkc == 1) {
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) store(nb, u, mb, v, acc[u][mb][v], scale[u], bias[u]);
    } else {
      constexpr int NV = NI * MB * 4;  // sums per lane
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(wave * NV + (u * MB + mb) * 4 + v) * 64 + lane] = acc[u][mb][v];
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int idx = (u * MB + mb) * 4 + v;
            if (idx % wkc == wk) {
              float sum = 0.0f;
              for (int j = 0; j < wkc; ++j) sum += red[((wn * wkc + j) * NV + idx) * 64 + lane];
              store(nb, u, mb, v, sum, scale[u], bias[u]);
            }
          }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < NI; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[u][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // 2. whole rounds of D steps; every step issues the loads of the step D
  //    later (the same instructions on every path), computes if it is one of
  //    the workgroup's steps inside the slice, and closes its column block
  //    after its last step.  T and the block ends are the same for every
  //    wave of the workgroup, so the barriers of finish() pair up.
  int ci = 0, cs = 0;  // compute position
  const int TR = (T + D - 1) / D * D;
  for (int t0 = 0; t0 < TR; t0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const bool run = t0 + j < T;
      const int sidx = wk * spw + cs;
      if (run && sidx < sps) compute(ring[j], sidx);
      float bias[NI], scale[NI];
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        bias[u] = HASB ? ring[j].b[u] : 0.0f;
        scale[u] = PERCH ? ring[j].s[u] : 0.0f;
      }
      const bool last = run && cs == spw - 1;
      const int cblk = ci;
      __builtin_amdgcn_sched_barrier(0);
      issue(ii, is, ring[j]);
      if (++is == spw) { is = 0; ++ii; }
      __builtin_amdgcn_sched_barrier(0);
      if (run && ++cs == spw) { cs = 0; ++ci; }
      if (last) finish(cblk, scale, bias);
    }
  }
  // the ring's last loads (past the end) are drained before the wave exits
  sk_wait_vmcnt<0>();
}

template <int ORDER, int SC, bool S16, bool HASB, int MB, int NI>
hipError_t launch_sk(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  auto kern = gemm_skinny_kernel<ORDER, SC, S16, HASB, MB, NI>;
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

// (two column blocks per wave: measured on MI355X, four were slower on
// every Llama-shaped projection and on the lm_head, by 5-70%)
template <int ORDER, int SC, bool S16, bool HASB>
hipError_t launch_sk_m(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  if (pl.ni != 2) return hipErrorInvalidValue;
  return pl.mb == 1 ? launch_sk<ORDER, SC, S16, HASB, 1, 2>(p, pl, s)
                    : launch_sk<ORDER, SC, S16, HASB, 2, 2>(p, pl, s);
}

template <int ORDER, int SC, bool S16>
hipError_t launch_sk_b(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  return p.bias ? launch_sk_m<ORDER, SC, S16, true>(p, pl, s)
                : launch_sk_m<ORDER, SC, S16, false>(p, pl, s);
}

template <int ORDER, int SC>
hipError_t launch_sk_s(const GemmParams& p, const SkinnyPlan& pl, hipStream_t s) {
  return p.scales16 ? launch_sk_b<ORDER, SC, true>(p, pl, s) : launch_sk_b<ORDER, SC, false>(p, pl, s);
}

}  // namespace

template <int ORDER>
hipError_t launch_skinny_kernels(const GemmParams& p, const SkinnyPlan& pl, bool perch,
                                 hipStream_t s) {
  if (perch) return launch_sk_s<ORDER, SC_CHANNEL>(p, pl, s);
  if (p.log2_gs >= 7) return launch_sk_s<ORDER, SC_STEP>(p, pl, s);
  return p.K % 32 == 0 ? launch_sk_s<ORDER, SC_ELEM>(p, pl, s)
                       : launch_sk_s<ORDER, SC_ELEM_KT>(p, pl, s);
}

}  // namespace q4
