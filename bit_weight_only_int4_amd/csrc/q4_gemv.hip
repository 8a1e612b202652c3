// q4_gemv.hip -- streaming fp32 GEMV for gfx950 (the decode regime, M = 1;
// also every activation row of Q4_MATH_F32).
//
// out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8) (+ bias[n]),
// the weight-only 4-bit linear of page 3 (#20943) and page 5; at M = 1 each
// token streams the whole weight once (page 4, "Kernel level").  The pages'
// decode schedule (page 4, "Why (8, 16)": several rows per workgroup and a
// short reduction) is prior art; this kernel is laid out for wave64 and HBM3E:
//
//  * A wave owns a 2048-wide span of K: lane l holds the chunk of 32
//    consecutive k at 32*l, so one wave-wide 128-bit load reads 1 KiB of one
//    weight row and no two lanes of a wave read the same activations.  A
//    workgroup has one wave per span (up to 8; longer K is split over
//    grid.z) times max(1, 4 / spans) row groups of R rows (2, 4 or 8, by
//    a measured rule in plan_gemv); the spans' partial sums meet in LDS.
//  * The workgroup's activations are read from HBM/L2 once, by buffer loads
//    that write LDS directly, and shared by its row groups (every wave
//    reading the same few KiB of activations from L2 would load the same
//    cache lines thousands of times per call).  Each lane issues its scale
//    and weight loads before it waits for the activations, so the
//    latencies overlap.
//  * Grouped scales are [G, N] row-major, so one row's scales lie N apart;
//    each lane reads the scales of its chunk's group for the R consecutive
//    rows of the workgroup, one 16-byte load per four rows.
//  * Interior tiles (all rows < N, all chunks inside K) run without per-lane
//    checks; only edge tiles take the guarded code.
//  * Unpack is branch-free: v_and_or_b32 builds binary16 (1024 + q) and
//    (64 + q), one v_pk_add_f16 per pair gives the exact c = q - 8, and
//    v_fma_mix_f32 multiplies c by the fp32 activation into an fp32 sum (no
//    binary16 rounding touches x or the products: the path is pure fp32).
//    A chunk's partial sum is scaled once (group_size a power of two from 32
//    to 2048), or each weight is RN32(c * s) (any other group_size);
//    per-channel scales multiply the finished dot product.
//  * The 64-lane sum uses DPP row operations; span waves are then added in
//    order, so results are deterministic.  With K split over grid.z the
//    partial sums go to the workspace and a second kernel adds them in split
//    order.
#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

enum ScaleMode : int { kPerChannel = 0, kStaged = 1, kGeneric = 2 };

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4
// and lgkmcnt 11:8 left free)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// a wave-uniform pointer in scalar registers (a buffer resource lives in
// SGPRs)
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// LDS slot (16 bytes) of floats 4v .. 4v+3 of lane l's 32-k chunk of span
// wk: the XOR with bits 1..3 of the lane puts the 16 lanes of one
// ds_read_b128 group on 16 distinct 4-bank groups.
__device__ __forceinline__ int x_slot(int wk, int l, int v) {
  return wk * 512 + l * 8 + (v ^ ((l >> 1) & 7));
}


template <bool QA4>
__device__ __forceinline__ void load_chunk(const uint8_t* row, int64_t byte0,
                                           int64_t row_bytes, bool full,
                                           uint32_t (&w)[4]) {
  if (full && QA4) {
    // streamed once per call: a non-temporal load, so the weights do not
    // displace cached lines that are reused (scales, activations); measured
    // faster on MI355X when the weights do not fit in the caches
    const u32x4_a4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(row + byte0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    return;
  }
  // unaligned rows, or the ragged end of a row: byte loads; bytes past the
  // row become 0x88 (c = 0) and meet zero activations
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t o = byte0 + 4 * d + b;
      const uint32_t byte = (full || o < row_bytes) ? (uint32_t)row[o] : 0x88u;
      v |= byte << (8 * b);
    }
    w[d] = v;
  }
}

// sum_k x * c over one 32-k chunk (four packed words), fp32 throughout
template <int ORDER>
__device__ __forceinline__ float chunk_dot(const uint32_t (&q)[4], const float (&x)[32],
                                           const Magic& mg) {
  float part[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h2 c[4];
    unpack_word(q[d], mg, c);
    float a = 0.0f;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      a = __builtin_fmaf((float)c[pp].x, x[8 * d + pair_k<ORDER>(pp, 0)], a);
      a = __builtin_fmaf((float)c[pp].y, x[8 * d + pair_k<ORDER>(pp, 1)], a);
    }
    part[d] = a;
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// same with a per-weight scale, w = RN32(c * s(k))
template <int ORDER>
__device__ __forceinline__ float chunk_dot_generic(const uint32_t (&q)[4], const float (&x)[32],
                                                   const Magic& mg, const float* scol,
                                                   int64_t lds, int64_t gs, int64_t G,
                                                   int64_t k0, bool valid) {
  float part[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h2 c[4];
    unpack_word(q[d], mg, c);
    float a = 0.0f;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ko = 8 * d + pair_k<ORDER>(pp, h);
        int64_t g = (k0 + ko) / gs;
        g = g < G - 1 ? g : G - 1;
        const float s = valid ? scol[g * lds] : 0.0f;
        const float w = (float)(h == 0 ? c[pp].x : c[pp].y) * s;
        a = __builtin_fmaf(w, x[ko], a);
      }
    part[d] = a;
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// Sum over the 64 lanes of a wave with DPP row operations (quad swaps, half
// row and row mirrors, then the gfx9 row broadcasts); lane 63 ends with the
// total, which is returned wave-uniform.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_take(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_take<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_take<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_take<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_take<0x140, 0xF>(v);  // row_mirror
  v += dpp_take<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_take<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One wave's tile: R rows x its 2048*CPL-wide K span.  GUARD = false is the
// interior case (every row < N, every chunk inside K): no per-lane checks.
// Loads are issued in the order they are consumed (activations, scales,
// then the weight rows one by one) and vector loads retire in order, so the
// arithmetic of row r overlaps the arrival of rows r+1 .. R-1.
//
// XL: the workgroup's activations arrive in LDS (xs, laid out by x_slot) by
// buffer loads the kernel issued before this call; the lane issues its
// scale and weight loads, then waits for all of them, meets the other
// waves and reads its chunk from LDS.
template <int CPL, int R, int ORDER, int SMODE, bool QA4, bool SA16, bool GUARD, bool XL>
__device__ __forceinline__ void gemv_tile(const GemvParams& p, int64_t m, int64_t n0,
                                          int64_t kspan, int64_t kz1, int lane,
                                          const float* xs, int wk, float (&acc)[R]) {
  const int64_t row_bytes = (p.K + 1) >> 1;
  int64_t k0[CPL];
  bool kfull[CPL], kany[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    k0[t] = kspan + 32 * (t * 64 + lane);
    kfull[t] = !GUARD || k0[t] + 32 <= kz1;
    kany[t] = !GUARD || k0[t] < kz1;
  }
  // activations of this lane's chunks
  float xr[CPL][32];
  const float* xrow = p.x + m * p.ldx;
#pragma unroll
  for (int t = 0; t < CPL && !XL; ++t) {
    if (kfull[t]) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const f32x4_a4 xv = *reinterpret_cast<const f32x4_a4*>(xrow + k0[t] + 4 * v);
        xr[t][4 * v + 0] = xv.x; xr[t][4 * v + 1] = xv.y;
        xr[t][4 * v + 2] = xv.z; xr[t][4 * v + 3] = xv.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) xr[t][i] = (k0[t] + i < kz1) ? xrow[k0[t] + i] : 0.0f;
    }
  }
  // grouped scales: the R consecutive rows of this chunk's group, one
  // 16-byte load per four rows when aligned
  float sv[CPL][R];
  if (SMODE == kStaged) {
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int64_t g = k0[t] >> p.log2_gs;
      const float* srow = p.scales + (kany[t] ? g : 0) * p.lds + n0;
      if (SA16 && !GUARD) {
#pragma unroll
        for (int r4 = 0; r4 < R; r4 += 4) {
          const f32x4_a4 v = *reinterpret_cast<const f32x4_a4*>(srow + r4);
          sv[t][r4 + 0] = v.x; sv[t][r4 + 1] = v.y; sv[t][r4 + 2] = v.z; sv[t][r4 + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
          sv[t][r] = (kany[t] && (!GUARD || n0 + r < p.N)) ? srow[r] : 0.0f;
      }
    }
  }
  // packed weights: R rows x CPL 16-byte loads, all in flight together
  uint32_t qv[R][CPL][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool rowok = !GUARD || n0 + r < p.N;
    const uint8_t* qrow = p.qw + (rowok ? n0 + r : 0) * p.ldq;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      if (rowok && kany[t]) {
        load_chunk<QA4>(qrow, k0[t] >> 1, row_bytes, kfull[t], qv[r][t]);
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) qv[r][t][d] = 0x88888888u;
      }
    }
  }
  if (XL) {
    static_assert(!XL || CPL == 1, "activations in LDS: one chunk per lane");
    // Wait for every load in flight: the activation loads and the scale and
    // weight loads above, issued together, so the wait is about one memory
    // latency.  (A partial count would depend on how the compiler merges
    // adjacent loads.)
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f4 xv = *reinterpret_cast<const f4*>(xs + 4 * x_slot(wk, lane, v));
      xr[0][4 * v + 0] = xv.x; xr[0][4 * v + 1] = xv.y;
      xr[0][4 * v + 2] = xv.z; xr[0][4 * v + 3] = xv.w;
    }
  }
  const Magic mg = Magic::make();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float a = 0.0f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      if (SMODE == kGeneric) {
        const int64_t n = n0 + r;
        const bool ok = (!GUARD || n < p.N) && kany[t];
        a += chunk_dot_generic<ORDER>(qv[r][t], xr[t], mg, p.scales + (ok ? n : 0), p.lds,
                                      p.group_size, p.G, k0[t], ok);
      } else if (SMODE == kStaged) {
        a = __builtin_fmaf(sv[t][r], chunk_dot<ORDER>(qv[r][t], xr[t], mg), a);
      } else {
        a += chunk_dot<ORDER>(qv[r][t], xr[t], mg);
      }
    }
    acc[r] = a;
  }
}

// Workgroup: WK waves along K (one per 2048*CPL span) times WR row groups of
// R rows (p.waves_k, p.waves_r; WK * WR <= 8).  XL: the workgroup's
// activations for its K range are brought into LDS once (dynamic LDS,
// WK x 8 KiB) and shared by its WR row groups.
template <int CPL, int R, int ORDER, int SMODE, bool QA4, bool SA16, bool XL>
__global__ void __launch_bounds__(512)
gemv_f32_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float red[8 * 8 * 8];
  constexpr int SPAN = 64 * CPL * 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave = wk * WR + wr; WR (row groups) is 1, 2 or 4
  const int WK = p.waves_k, WR = p.waves_r, W = WK * WR;
  const int lwr = WR == 4 ? 2 : WR == 2 ? 1 : 0;
  const int wr = wave & (WR - 1), wk = wave >> lwr;
  const int64_t m = blockIdx.y;
  const int z = blockIdx.z;
  const int64_t n0 = ((int64_t)xcd_swizzle(blockIdx.x, gridDim.x) * WR + wr) * R;
  const int64_t kz0 = (int64_t)z * p.k_per_split;
  const int64_t kz1 = (kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K;
  const int64_t kspan = kz0 + (int64_t)wk * SPAN;

  if (XL) {
    // activations [kz0, kz1) of row m: WK * 8 wave loads of 1 KiB, spread
    // over the W waves; reads past kz1 return zeros.  Issued before the
    // weight loads: measured faster here (in the low-batch kernel, after).
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(uniform_ptr(p.x + m * p.ldx + kz0)), (short)0,
        (int)((kz1 - kz0) * 4), 0x00020000);
    for (int i = wave; i < WK * 8; i += W) {
      const int j = i * 64 + lane;
      const int span = j >> 9, l = (j >> 3) & 63, v = (j & 7) ^ ((l >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_ptr_t)((char*)xs + i * 1024), 16,
          (uint32_t)((span * 2048 + 32 * l + 4 * v) * 4), 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  }

  float acc[R];
  if (n0 + R <= p.N && kspan + SPAN <= kz1)
    gemv_tile<CPL, R, ORDER, SMODE, QA4, SA16, false, XL>(p, m, n0, kspan, kz1, lane, xs, wk, acc);
  else
    gemv_tile<CPL, R, ORDER, SMODE, QA4, SA16, true, XL>(p, m, n0, kspan, kz1, lane, xs, wk, acc);

#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
  if (WK > 1) {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) red[(wr * 8 + wk) * 8 + r] = acc[r];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v = red[(wr * 8 + 0) * 8 + r];
      for (int w = 1; w < WK; ++w) v += red[(wr * 8 + w) * 8 + r];
      acc[r] = v;
    }
  }
  // lane r of the row group's first wave stores row n0 + r
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t n = n0 + r;
    if (lane != r || n >= p.N) continue;
    float v = acc[r];
    if (SMODE == kPerChannel) v *= p.scales[n];
    if (p.split > 1) {
      p.partial[((int64_t)z * p.M + m) * p.N + n] = v;
    } else {
      if (p.bias) v += p.bias[n];
      p.out[m * p.ldo + n] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Low batch: MB activation rows per workgroup (2 <= M, MB in {2, 4, 8}),
// weights streamed once for all of them.  Activations reach LDS as in the
// XL kernel (one slice per row, MB * WK * 8 KiB); each lane unpacks its R
// weight chunks once and applies them to every row, still pure fp32.
// Staged or per-channel scales, dword-aligned weight rows, K % 4 == 0.
// ---------------------------------------------------------------------------
template <int R, int ORDER, int SMODE, bool SA16, int MB>
__global__ void __launch_bounds__(512)
gemv_lb_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float red[8 * 8 * MB * R];
  constexpr int SPAN = 2048;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave = wk * WR + wr; WR (row groups) is 1, 2 or 4
  const int WK = p.waves_k, WR = p.waves_r, W = WK * WR;
  const int lwr = WR == 4 ? 2 : WR == 2 ? 1 : 0;
  const int wr = wave & (WR - 1), wk = wave >> lwr;
  const int64_t m0 = (int64_t)blockIdx.y * MB;
  const int z = blockIdx.z;
  const int64_t n0 = ((int64_t)xcd_swizzle(blockIdx.x, gridDim.x) * WR + wr) * R;
  const int64_t kz0 = (int64_t)z * p.k_per_split;
  const int64_t kz1 = (kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K;
  const int64_t kspan = kz0 + (int64_t)wk * SPAN;
  const int64_t k0 = kspan + 32 * lane;
  const bool kany = k0 < kz1, kfull = k0 + 32 <= kz1;
  const bool interior = n0 + R <= p.N && kspan + SPAN <= kz1;

  // scales of this chunk's group for the R rows
  float sv[R];
  if (SMODE == kStaged) {
    const int64_t g = k0 >> p.log2_gs;
    const float* srow = p.scales + (kany ? g : 0) * p.lds + n0;
    if (SA16 && interior) {
#pragma unroll
      for (int r4 = 0; r4 < R; r4 += 4) {
        const f32x4_a4 v = *reinterpret_cast<const f32x4_a4*>(srow + r4);
        sv[r4 + 0] = v.x; sv[r4 + 1] = v.y; sv[r4 + 2] = v.z; sv[r4 + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) sv[r] = (kany && n0 + r < p.N) ? srow[r] : 0.0f;
    }
  }
  // packed weights, R rows x one 32-k chunk
  const int64_t row_bytes = (p.K + 1) >> 1;
  uint32_t qv[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (n0 + r < p.N && kany) {
      load_chunk<true>(p.qw + (n0 + r) * p.ldq, k0 >> 1, row_bytes, kfull, qv[r]);
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) qv[r][d] = 0x88888888u;
    }
  }
  // then the activations of rows m0 .. m0 + MB - 1 (those < M), [kz0, kz1) each
  for (int i = wave; i < MB * WK * 8; i += W) {
    const int m = i / (WK * 8), ii = i % (WK * 8);
    if (m0 + m >= p.M) continue;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(uniform_ptr(p.x + (m0 + m) * p.ldx + kz0)), (short)0,
        (int)((kz1 - kz0) * 4), 0x00020000);
    const int j = ii * 64 + lane;
    const int span = j >> 9, l = (j >> 3) & 63, v = (j & 7) ^ ((l >> 1) & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)((char*)xs + i * 1024), 16,
                                             (uint32_t)((span * 2048 + 32 * l + 4 * v) * 4),
                                             0, 0, 0);
  }
  asm volatile("" ::: "memory");
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // unpack once
  const Magic mg = Magic::make();
  h2 c[R][4][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int d = 0; d < 4; ++d) unpack_word(qv[r][d], mg, c[r][d]);

  float acc[MB][R];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
    if (m0 + m >= p.M) continue;
    float xr[32];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f4 xv = *reinterpret_cast<const f4*>(xs + (size_t)m * WK * 2048 +
                                                   4 * x_slot(wk, lane, v));
      xr[4 * v + 0] = xv.x; xr[4 * v + 1] = xv.y; xr[4 * v + 2] = xv.z; xr[4 * v + 3] = xv.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float part[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float a = 0.0f;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          a = __builtin_fmaf((float)c[r][d][pp].x, xr[8 * d + pair_k<ORDER>(pp, 0)], a);
          a = __builtin_fmaf((float)c[r][d][pp].y, xr[8 * d + pair_k<ORDER>(pp, 1)], a);
        }
        part[d] = a;
      }
      const float dot = (part[0] + part[1]) + (part[2] + part[3]);
      acc[m][r] = SMODE == kStaged ? sv[r] * dot : dot;
    }
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_sum(acc[m][r]);
  if (WK > 1) {
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) red[((wr * 8 + wk) * MB + m) * R + r] = acc[m][r];
    }
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float v = red[((wr * 8 + 0) * MB + m) * R + r];
        for (int w2 = 1; w2 < WK; ++w2) v += red[((wr * 8 + w2) * MB + m) * R + r];
        acc[m][r] = v;
      }
  }
  // lane m * R + r stores (m0 + m, n0 + r)
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t mm = m0 + m, n = n0 + r;
      if (lane != m * R + r || mm >= p.M || n >= p.N) continue;
      float v = acc[m][r];
      if (SMODE == kPerChannel) v *= p.scales[n];
      if (p.split > 1) {
        p.partial[((int64_t)z * p.M + mm) * p.N + n] = v;
      } else {
        if (p.bias) v += p.bias[n];
        p.out[mm * p.ldo + n] = v;
      }
    }
}

}  // namespace

__global__ void splitk_reduce_kernel(const float* __restrict__ partial,
                                     const float* __restrict__ bias,
                                     float* __restrict__ out, int64_t ldo,
                                     int64_t M, int64_t N, int split) {
  // four consecutive outputs per thread when the rows allow 16-byte access
  const bool vec = (N % 4 == 0) && (ldo % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec) {
    const int64_t e = 4 * idx;
    if (e >= M * N) return;
    const int64_t m = e / N, n = e % N;
    float4 v = *reinterpret_cast<const float4*>(partial + e);
    for (int z = 1; z < split; ++z) {
      const float4 w = *reinterpret_cast<const float4*>(partial + (int64_t)z * M * N + e);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    if (bias) { v.x += bias[n]; v.y += bias[n + 1]; v.z += bias[n + 2]; v.w += bias[n + 3]; }
    *reinterpret_cast<float4*>(out + m * ldo + n) = v;
    return;
  }
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float v = partial[idx];
  for (int z = 1; z < split; ++z) v += partial[(int64_t)z * M * N + idx];
  if (bias) v += bias[n];
  out[m * ldo + n] = v;
}

hipError_t launch_splitk_reduce(const float* partial, const float* bias, float* out, int64_t ldo,
                                int64_t M, int64_t N, int split, hipStream_t s) {
  const bool vec = (N % 4 == 0) && (ldo % 4 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  const int64_t threads = vec ? (M * N) / 4 : M * N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, partial, bias, out, ldo, M, N, split);
  return hipGetLastError();
}

// ---- host-side plan and launch ---------------------------------------------

namespace {

int scale_mode(int64_t gs, int64_t K) {
  if (gs == 0 || gs >= K) return kPerChannel;
  const bool pow2 = (gs & (gs - 1)) == 0;
  if (pow2 && gs >= 32 && gs <= 2048) return kStaged;
  return kGeneric;
}

template <int R, int ORDER, int SMODE, bool QA4, bool SA16>
hipError_t launch_t(const GemvParams& p, dim3 grid, bool xl, hipStream_t s) {
  const int nwaves = p.waves_k * p.waves_r;
  if (xl)
    hipLaunchKernelGGL((gemv_f32_kernel<1, R, ORDER, SMODE, QA4, SA16, true>), grid,
                       dim3(64 * nwaves), (size_t)p.waves_k * 8192, s, p);
  else
    hipLaunchKernelGGL((gemv_f32_kernel<1, R, ORDER, SMODE, QA4, SA16, false>), grid,
                       dim3(64 * nwaves), 0, s, p);
  return hipGetLastError();
}

template <int R, int ORDER, int SMODE, bool SA16, int MB>
hipError_t launch_lb_t(const GemvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemv_lb_kernel<R, ORDER, SMODE, SA16, MB>), grid,
                     dim3(64 * p.waves_k * p.waves_r), (size_t)MB * p.waves_k * 8192, s, p);
  return hipGetLastError();
}

template <int R, int MB>
hipError_t launch_lb_r(const GemvParams& p, dim3 grid, int order, int smode, bool sa16,
                       hipStream_t s) {
#define Q4_LB_CASE(O, S, B) \
  if (order == O && smode == S && sa16 == B) return launch_lb_t<R, O, S, B, MB>(p, grid, s);
  Q4_LB_CASE(0, 0, false) Q4_LB_CASE(1, 0, false)
  Q4_LB_CASE(0, 1, false) Q4_LB_CASE(1, 1, false)
  Q4_LB_CASE(0, 1, true) Q4_LB_CASE(1, 1, true)
#undef Q4_LB_CASE
  return hipErrorInvalidValue;
}

template <int MB>
hipError_t launch_lb(const GemvParams& p, dim3 grid, int R, int order, int smode, bool sa16,
                     hipStream_t s) {
  return R == 8   ? launch_lb_r<8, MB>(p, grid, order, smode, sa16, s)
         : R == 4 ? launch_lb_r<4, MB>(p, grid, order, smode, sa16, s)
                  : launch_lb_r<2, MB>(p, grid, order, smode, sa16, s);
}

template <int R>
hipError_t launch_r(const GemvParams& p, dim3 grid, bool xl, int order, int smode, bool qa4,
                    bool sa16, hipStream_t s) {
#define Q4_GEMV_CASE(O, S, A, B) \
  if (order == O && smode == S && qa4 == A && sa16 == B) return launch_t<R, O, S, A, B>(p, grid, xl, s);
  Q4_GEMV_CASE(0, 0, true, false) Q4_GEMV_CASE(0, 2, true, false)
  Q4_GEMV_CASE(1, 0, true, false) Q4_GEMV_CASE(1, 2, true, false)
  Q4_GEMV_CASE(0, 0, false, false) Q4_GEMV_CASE(0, 2, false, false)
  Q4_GEMV_CASE(1, 0, false, false) Q4_GEMV_CASE(1, 2, false, false)
  Q4_GEMV_CASE(0, 1, true, true) Q4_GEMV_CASE(0, 1, true, false)
  Q4_GEMV_CASE(1, 1, true, true) Q4_GEMV_CASE(1, 1, true, false)
  Q4_GEMV_CASE(0, 1, false, true) Q4_GEMV_CASE(0, 1, false, false)
  Q4_GEMV_CASE(1, 1, false, true) Q4_GEMV_CASE(1, 1, false, false)
#undef Q4_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace

// Activation rows per workgroup of the low-batch kernel: the next power of
// two >= M, at most 8 and at most 8 / spans (its LDS holds MB x spans x 8 KiB
// of activations); 1 selects the one-row kernel.
static int lowbatch_rows(int64_t M, int waves_k) {
  if (M < 2) return 1;
  int cap = 8 / waves_k;
  if (cap < 2) return 1;
  int mb = 2;
  while (mb < M && mb < cap) mb *= 2;
  return mb;
}

int gemv_lowbatch_max_rows(int64_t K) {
  const int64_t spans = (K + 2047) / 2048;
  const int64_t split = (spans + 7) / 8;
  const int waves_k = (int)((spans + split - 1) / split);
  const int cap = 8 / waves_k;
  return cap >= 2 ? cap : 1;
}

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  (void)group_size;
  GemvPlan pl{};
  pl.cfg = 1;  // one chunk of 32 k per lane; a wave spans 2048 k
  const int64_t spans = (K + 2047) / 2048;
  pl.split = (int)((spans + 7) / 8);  // at most 8 span-waves per workgroup
  pl.waves_k = (int)((spans + pl.split - 1) / pl.split);
  pl.k_per_split = (int64_t)pl.waves_k * 2048;
  // Rows per wave and row groups per workgroup, from a sweep on MI355X over
  // the Llama-shaped projections: about four waves per workgroup, four rows
  // per wave unless that leaves fewer than 2048 waves (then two), eight
  // only for deep K (more than four spans) where eight still give 2048.
  pl.mb = lowbatch_rows(M, pl.waves_k);
  const int64_t mrows = (M + pl.mb - 1) / pl.mb;  // activation row blocks
  auto waves = [&](int r) { return ((N + r - 1) / r) * pl.waves_k * pl.split * mrows; };
  int rows = 4;
  if (waves(4) < 2048) rows = 2;
  if (pl.waves_k > 4 && waves(8) >= 2048) rows = 8;
  pl.rows_per_wave = rows;
  int wr = 4 / pl.waves_k;
  if (wr < 1) wr = 1;
  while (wr > 1 && (int64_t)(wr / 2) * rows >= N) wr /= 2;
  pl.waves_r = wr;
  pl.rows_per_block = rows * wr;
  pl.blocks_n = (N + pl.rows_per_block - 1) / pl.rows_per_block;
  return pl;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  const GemvPlan pl = plan_gemv(M, N, K, group_size);
  return pl.split > 1 ? (size_t)pl.split * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemv(const GemvParams& p0, int order, bool qa4, hipStream_t s) {
  GemvParams p = p0;
  const GemvPlan pl = plan_gemv(p.M, p.N, p.K, p.group_size);
  p.k_per_split = pl.k_per_split;
  p.split = pl.split;
  p.waves_k = pl.waves_k;
  // activations through LDS when every 16-byte piece of the row range is
  // whole or wholly past its end (K % 4 == 0); else one row group per
  // workgroup, each wave reading its activations itself
  const bool xl = p.K % 4 == 0;
  p.waves_r = xl ? pl.waves_r : 1;
  const int64_t rpb = (int64_t)pl.rows_per_wave * p.waves_r;
  const int smode = scale_mode(p.group_size, p.K);
  if (smode == kPerChannel) p.group_size = 0;  // one group: scale row 0 per channel
  int l2 = 0;
  if (smode == kStaged)
    while ((1LL << l2) < p.group_size) ++l2;
  p.log2_gs = l2;
  const int R = pl.rows_per_wave;
  // four consecutive scales per 16-byte load: needs 16-byte aligned rows of
  // the scale matrix (each row group starts at a multiple of R >= 4)
  const bool sa16 = smode == kStaged && R >= 4 &&
                    (reinterpret_cast<uintptr_t>(p.scales) % 16 == 0) && (p.lds % 4 == 0);
  p.rows_per_block = (int32_t)rpb;
  // several activation rows per workgroup (weights read once for all):
  // aligned weights, activations through LDS, staged or per-channel scales
  const int mb = (xl && qa4 && smode != kGeneric) ? pl.mb : 1;
  hipError_t e;
  if (mb > 1) {
    const dim3 grid((unsigned)((p.N + rpb - 1) / rpb), (unsigned)((p.M + mb - 1) / mb),
                    (unsigned)pl.split);
    e = mb == 8   ? launch_lb<8>(p, grid, R, order, smode, sa16, s)
        : mb == 4 ? launch_lb<4>(p, grid, R, order, smode, sa16, s)
                  : launch_lb<2>(p, grid, R, order, smode, sa16, s);
  } else {
    const dim3 grid((unsigned)((p.N + rpb - 1) / rpb), (unsigned)p.M, (unsigned)pl.split);
    e = R == 8   ? launch_r<8>(p, grid, xl, order, smode, qa4, sa16, s)
        : R == 4 ? launch_r<4>(p, grid, xl, order, smode, qa4, sa16, s)
                 : launch_r<2>(p, grid, xl, order, smode, qa4, sa16, s);
  }
  if (e != hipSuccess || pl.split == 1) return e;
  return launch_splitk_reduce(p.partial, p.bias, p.out, p.ldo, p.M, p.N, p.split, s);
}

}  // namespace q4
