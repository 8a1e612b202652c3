// q4_gemv_kernels.h -- the fp32 GEMV kernels (q4_gemv.hip describes the
// design), templated on the scale element type ST: float, or _Float16 for
// binary16 scales (q4f16_1 weights, widened exactly).  Each scale type is
// compiled in its own translation unit (q4_gemv_s32.hip, q4_gemv_s16.hip),
// which instantiates launch_gemv_kernels<ST>; the plan and the choice of
// kernel stay in q4_gemv.hip.  Not part of the public ABI.
#pragma once

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

using namespace gemv;

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

// R consecutive scales from element sb on (R a multiple of 4), four per
// vector load: 16 bytes of fp32 or 8 bytes of binary16 (widened exactly).
// The caller guarantees sb * sizeof(ST) is a multiple of that load.
template <int R, typename ST>
__device__ __forceinline__ void load_scales4(const ST* sp, int64_t sb, float (&sv)[R]) {
#pragma unroll
  for (int r4 = 0; r4 < R; r4 += 4) {
    if constexpr (sizeof(ST) == 2) {
      const h4 v = *reinterpret_cast<const h4*>(sp + sb + r4);
      sv[r4 + 0] = (float)v.x; sv[r4 + 1] = (float)v.y;
      sv[r4 + 2] = (float)v.z; sv[r4 + 3] = (float)v.w;
    } else {
      const f32x4_a4 v = *reinterpret_cast<const f32x4_a4*>(sp + sb + r4);
      sv[r4 + 0] = v.x; sv[r4 + 1] = v.y; sv[r4 + 2] = v.z; sv[r4 + 3] = v.w;
    }
  }
}

// the scale array of a call: fp32, or binary16 (q4f16_1 weights)
template <typename ST>
__device__ __forceinline__ const ST* scale_ptr(const GemvParams& p) {
  if constexpr (sizeof(ST) == 2) return p.scales16;
  else return p.scales;
}

// sum_k x * c over one 32-k chunk (four packed words), fp32 throughout.
// Each word's eight products are summed in k-pair order into their own
// partial; the four partials' chains are issued interleaved (word innermost),
// so consecutive FMAs never depend on each other.
template <int ORDER>
__device__ __forceinline__ float chunk_dot(const uint32_t (&q)[4], const float (&x)[32],
                                           const Magic& mg) {
  h2 c[4][4];
#pragma unroll
  for (int d = 0; d < 4; ++d) unpack_word(q[d], mg, c[d]);
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int h = 0; h < 2; ++h)
    {
#pragma unroll
      for (int d = 0; d < 4; ++d)
        part[d] = __builtin_fmaf((float)(h == 0 ? c[d][pp].x : c[d][pp].y),
                                 x[8 * d + pair_k<ORDER>(pp, h)], part[d]);
      // keep the four chains interleaved (the scheduler would otherwise
      // issue them one after another)
      __builtin_amdgcn_sched_barrier(0);
    }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// same with a per-weight scale, w = RN32(c * s(k))
template <int ORDER, typename ST>
__device__ __forceinline__ float chunk_dot_generic(const uint32_t (&q)[4], const float (&x)[32],
                                                   const Magic& mg, const ST* sp, int64_t col,
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
        const float s = valid ? (float)sp[g * lds + col] : 0.0f;
        const float w = (float)(h == 0 ? c[pp].x : c[pp].y) * s;
        a = __builtin_fmaf(w, x[ko], a);
      }
    part[d] = a;
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// ---------------------------------------------------------------------------
// Integer inner products for the streaming GEMV.  A lane's 32-k activation
// chunk is written as block fixed point: with E the binary exponent of the
// chunk's largest |x| (2^(E-1) <= max |x| < 2^E), X_k = RN(x_k 2^(26 - E)),
// |X_k| <= 2^26, i.e. 27 significant bits against the chunk's largest value.
// Each X_k is split into seven balanced base-16 digits (-8..7, X_k =
// sum_l d_l 16^l), stored as signed 4-bit fields, and the digits are
// transposed so that register lim[l][d] holds digit l of the eight x of word
// d in the nibble positions of that word's codes.  A packed word XOR 0x8 in
// every nibble is its codes c = q - 8 as signed 4-bit fields, so
// v_dot8_i32_i4 of the two gives sum over the word of c * d_l exactly; seven
// of them per word, integer sums over the chunk, and
//   sum_k c_k X_k = T_hi 2^16 + T_lo  (T_lo = sum_{l<4} S_l 16^l,
//   T_hi = sum_{l>=4} S_l 16^(l-4), both exact in fp32)
// is formed with one fp32 rounding and scaled by 2^(E - 26).  Per packed
// word: 1 XOR and 7 dot products, against 9 unpack and 8 FMA instructions.
// The chunk's largest |x| is taken over the bit patterns of |x|, where NaN
// ranks above inf; a non-finite largest |x| becomes the chunk's factor, so
// every row that meets the chunk gets a non-finite sum (inf or NaN; which
// one, and the sign of an inf, may differ from an fp32 sum over the same
// products).
// ---------------------------------------------------------------------------

// 8 x 8 transpose of 4-bit fields: afterwards R[l] nibble i = (before) R[i]
// nibble l.  Three exchange stages: 16-bit halves between rows i, i + 4;
// bytes between rows i, i + 2; nibbles between rows i, i + 1.
__device__ __forceinline__ void nibble_transpose(uint32_t (&R)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = R[i], b = R[i + 4];
    R[i] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    R[i + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = (t & 1) + 4 * (t >> 1);
    const uint32_t a = R[i], b = R[i + 2];
    R[i] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    R[i + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t a = R[i], b = R[i + 1];
    R[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    R[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// the chunk x (k order of the lane's 32 k) as digits lim and factor e
template <int ORDER>
__device__ __forceinline__ void chunk_digits(const float (&x)[32], uint32_t (&lim)[7][4],
                                             float& e) {
  uint32_t mb = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t a = __builtin_bit_cast(uint32_t, x[k]) & 0x7FFFFFFFu;
    mb = mb > a ? mb : a;
  }
  const float m = __builtin_bit_cast(float, mb);
  const int E = __builtin_amdgcn_frexp_expf(m);  // 0 for m = 0
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int X = (int)__builtin_rintf(__builtin_ldexpf(x[8 * d + nibble_k<ORDER>(i)], 26 - E));
      // balanced digits: nibble l of X + 0x08888888 is d_l + 8; XOR 8 gives
      // d_l as a signed 4-bit field
      R[i] = ((uint32_t)X + 0x08888888u) ^ 0x08888888u;
    }
    nibble_transpose(R);
#pragma unroll
    for (int l = 0; l < 7; ++l) lim[l][d] = R[l];
  }
  e = __builtin_isfinite(m) ? __builtin_ldexpf(1.0f, E - 26) : m;
}

// sum over one chunk of c_k X_k (four packed words), one fp32 rounding
__device__ __forceinline__ float chunk_dot_digits(const uint32_t (&q)[4],
                                                  const uint32_t (&lim)[7][4]) {
  int S[7] = {0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int c = (int)(q[d] ^ 0x88888888u);
#pragma unroll
    for (int l = 0; l < 7; ++l) S[l] = __builtin_amdgcn_sdot8(c, (int)lim[l][d], S[l], false);
  }
  const int lo = S[0] + 16 * (S[1] + 16 * (S[2] + 16 * S[3]));
  const int hi = S[4] + 16 * (S[5] + 16 * S[6]);
  return __builtin_fmaf((float)hi, 65536.0f, (float)lo);
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
template <int CPL, int R, int ORDER, int SMODE, bool QA4, bool SA16, bool GUARD, bool XL,
          typename ST>
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
      const int64_t sb = (kany[t] ? g : 0) * p.lds + n0;
      if (SA16 && !GUARD) {
        load_scales4<R>(scale_ptr<ST>(p), sb, sv[t]);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
          sv[t][r] = (kany[t] && (!GUARD || n0 + r < p.N))
                         ? (float)scale_ptr<ST>(p)[sb + r] : 0.0f;
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
    // Wait for the activation loads only (the kernel issued them before the
    // scale and weight loads, and vector memory operations retire in
    // order): vmcnt may still count the loads issued after them.  Interior
    // tiles of aligned rows issue exactly one 16-byte load per weight row
    // (rows lie ldq bytes apart, so none merge) and, for fp32 scales, one
    // 16-byte scale load per four rows; counting fewer than were issued only
    // waits longer, so binary16 and scalar scale loads, which the compiler
    // may merge, are not counted.  Each row's arithmetic then waits for its
    // own load alone (the compiler's wait), so the first rows are computed
    // while the later ones are still arriving.
    constexpr int NEWER =
        (!GUARD && QA4) ? R + ((SMODE == kStaged && SA16 && sizeof(ST) == 4) ? R / 4 : 0) : 0;
    asm volatile("" ::: "memory");
    wait_vmcnt<NEWER>();
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
        a += chunk_dot_generic<ORDER>(qv[r][t], xr[t], mg, scale_ptr<ST>(p), ok ? n : 0, p.lds,
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
template <int CPL, int R, int ORDER, int SMODE, bool QA4, bool SA16, bool XL, typename ST>
__global__ void __launch_bounds__(512)
gemv_f32_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float red[8 * 8 * 8];
  constexpr int SPAN = 64 * CPL * 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave = wk * WR + wr; WR (row groups) is a power of two
  const int WK = p.waves_k, WR = p.waves_r, W = WK * WR;
  const int lwr = 31 - __builtin_clz(WR);
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
    gemv_tile<CPL, R, ORDER, SMODE, QA4, SA16, false, XL, ST>(p, m, n0, kspan, kz1, lane, xs, wk,
                                                              acc);
  else
    gemv_tile<CPL, R, ORDER, SMODE, QA4, SA16, true, XL, ST>(p, m, n0, kspan, kz1, lane, xs, wk,
                                                             acc);

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
    if (SMODE == kPerChannel) v *= (float)scale_ptr<ST>(p)[n];
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
template <int R, int ORDER, int SMODE, bool SA16, int MB, typename ST>
__global__ void __launch_bounds__(512)
gemv_lb_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float red[8 * 8 * MB * R];
  constexpr int SPAN = 2048;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave = wk * WR + wr; WR (row groups) is a power of two
  const int WK = p.waves_k, WR = p.waves_r, W = WK * WR;
  const int lwr = 31 - __builtin_clz(WR);
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
    const int64_t sb = (kany ? g : 0) * p.lds + n0;
    if (SA16 && interior) {
      load_scales4<R>(scale_ptr<ST>(p), sb, sv);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
        sv[r] = (kany && n0 + r < p.N) ? (float)scale_ptr<ST>(p)[sb + r] : 0.0f;
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
      // each word's products in k-pair order into its own partial, the four
      // chains issued interleaved (as in chunk_dot)
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int d = 0; d < 4; ++d)
            part[d] = __builtin_fmaf((float)(h == 0 ? c[r][d][pp].x : c[r][d][pp].y),
                                     xr[8 * d + pair_k<ORDER>(pp, h)], part[d]);
          __builtin_amdgcn_sched_barrier(0);
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
      if (SMODE == kPerChannel) v *= (float)scale_ptr<ST>(p)[n];
      if (p.split > 1) {
        p.partial[((int64_t)z * p.M + mm) * p.N + n] = v;
      } else {
        if (p.bias) v += p.bias[n];
        p.out[mm * p.ldo + n] = v;
      }
    }
}


// ---------------------------------------------------------------------------
// Streaming GEMV: one activation row, dword-aligned weight rows, K a multiple
// of 32 and at most 8 spans of 2048, staged (power-of-two groups 32..2048)
// or per-channel scales.  Every row a wave owns is traversed over the whole
// of K by that wave, so no two waves meet to add partial sums:
//  * A workgroup of W waves (4 or 8) stages the activations [0, 2048 S) in
//    LDS once (zeros past K) and then loops over blocks of W * R
//    rows: block b = L + i * gridDim.x for its XCD-ordered index L, so the
//    blocks an XCD runs at once are neighbours and share the scale lines.
//  * Inside a block, wave w owns rows R w .. R w + R - 1 (R = 2 or 4).  A
//    wave step is one 2048-k span of its rows: lane l holds the 32 k at
//    32 l, one 16-byte load per row (1 KiB per wave-wide load,
//    non-temporal), and the scales of its chunk's group for all R rows in
//    one load.
//  * A ring of D wave steps (1 or 2): while one step computes, the loads of
//    the next D - 1 are in flight, and the wave issues the loads D steps
//    ahead before it adds up and stores the rows it has just finished.
//  * Loads go through buffer resources that cover exactly the caller's
//    arrays: past the last row (clamped) or the last scale they return zeros,
//    which meet zero activations past K.
// The arithmetic is that of gemv_f32_kernel (exact c, fp32 FMA chains, one
// scale multiply per 32-k chunk, per-channel scales after the sum), so the
// two give the same kind of fp32 result; their summation orders differ.
// ---------------------------------------------------------------------------
template <int R>
struct StreamSlot {
  uint32_t q[R][4];
  float s[R];  // grouped: this lane's chunk scale for each row
  float e;     // per-channel: lane r's row scale
  float b;     // bias: lane r's row bias
};

// the R (2 or 4) consecutive scales at byte offset off, one load (fp32: 8 or
// 16 bytes; binary16: 4 or 8 bytes, widened exactly)
template <int R, typename ST>
__device__ __forceinline__ void load_scale_row(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                               float (&s)[R]) {
  static_assert(R == 2 || R == 4, "two or four rows per wave step");
  typedef float f2v __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(ST) == 4 && R == 2) {
    const f2v v = __builtin_bit_cast(f2v, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
    s[0] = v.x; s[1] = v.y;
  } else if constexpr (sizeof(ST) == 4) {
    const f4 v = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
  } else if constexpr (R == 2) {
    const h2 v = __builtin_bit_cast(h2, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    s[0] = (float)v.x; s[1] = (float)v.y;
  } else {
    const h4 v = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
    s[0] = (float)v.x; s[1] = (float)v.y; s[2] = (float)v.z; s[3] = (float)v.w;
  }
}

template <typename ST>
__device__ __forceinline__ float load_scale_one(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(ST) == 4)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  else
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
}

template <int W, int R, int ORDER, bool PERCH, bool ONESPAN, bool HASB, int D, typename ST,
          bool IDOT = false>
__global__ void __launch_bounds__(64 * W)
gemv_stream_kernel(const GemvParams p) {
  static_assert(!IDOT || ONESPAN, "integer products: one span, digits formed once");
  constexpr uint32_t SB = sizeof(ST);
  extern __shared__ __attribute__((aligned(16))) float xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = ONESPAN ? 1 : p.spans;

  // 1. the activations [0, 2048 S) into LDS (x_slot layout), zeros past K:
  //    S * 8 wave-wide loads of 1 KiB spread over the waves
  {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(uniform_ptr(p.x)), (short)0, (int)(p.K * 4), 0x00020000);
    for (int i = wave; i < S * 8; i += W) {
      const int j = i * 64 + lane;
      const int span = j >> 9, l = (j >> 3) & 63, v = (j & 7) ^ ((l >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_ptr_t)((char*)xs + i * 1024), 16,
          (uint32_t)((span * 2048 + 32 * l + 4 * v) * 4), 0, 0, 0);
    }
  }

  // 2. this wave's steps: blocks L, L + G, ... (G = gridDim.x), S spans each
  const int G = (int)gridDim.x;
  const int L = (int)xcd_swizzle(blockIdx.x, gridDim.x);
  const int T = ((p.blocks - L + G - 1) / G) * S;
  const int64_t Kp = (p.K + 1) >> 1;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.qw), (short)0,
      (int)(uint32_t)((uint64_t)(p.N - 1) * (uint64_t)p.ldq + (uint64_t)Kp), 0x00020000);
  const ST* sp = scale_ptr<ST>(p);
  const uint64_t sbytes = PERCH ? (uint64_t)p.N * SB
                                : ((uint64_t)(p.G - 1) * (uint64_t)p.lds + (uint64_t)p.N) * SB;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<ST*>(sp), (short)0, (int)(uint32_t)sbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.bias), (short)0, (int)(p.N * 4), 0x00020000);
  const uint32_t qlane = 16u * (uint32_t)lane;
  // grouped: byte offset of this lane's chunk group in span 0, and per span
  uint32_t slane = 0, sspan = 0;
  if (!PERCH) {
    slane = (uint32_t)(((32 * lane) >> p.log2_gs) * p.lds) * SB;
    sspan = (uint32_t)((2048 >> p.log2_gs) * p.lds) * SB;
  }
  // The loads of step t (block i = t / S, span s = t % S).  Rows past N read
  // row N - 1; lane l's per-row values (per-channel scale, bias) are those of
  // row n0 + (l % R).  Steps past the wave's last one (issued so that every
  // step issues the same loads) read lines of the activation row instead,
  // spread over it and resident in L2: no weight traffic.
  const __amdgpu_buffer_rsrc_t rx2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(uniform_ptr(p.x)), (short)0, (int)(p.K * 4), 0x00020000);
  const uint32_t xspan = (uint32_t)(p.K * 4) & ~1023u;  // >= 1024: K >= 256 here
  const uint32_t dlane = ((uint32_t)(wave * 1024 + 16 * lane)) % (xspan ? xspan : 1024u);
  auto issue = [&](int t, StreamSlot<R>& sl) {
    const bool live = t < T;
    const int i = live ? t / S : 0, s = live ? t - i * S : 0;
    const int n0 = ((L + i * G) * W + wave) * R;
    const int nl = n0 + (lane & (R - 1)) < p.N ? n0 + (lane & (R - 1)) : (int)p.N - 1;
    const __amdgpu_buffer_rsrc_t rq_ = live ? rq : rx2;
    const __amdgpu_buffer_rsrc_t rs_ = live ? rs : rx2;
    const __amdgpu_buffer_rsrc_t rb_ = live ? rb : rx2;
    if (PERCH) sl.e = load_scale_one<ST>(rs_, live ? (uint32_t)nl * SB : dlane);
    else load_scale_row<R, ST>(rs_, live ? (uint32_t)s * sspan + (uint32_t)n0 * SB + slane : dlane, sl.s);
    if (HASB)
      sl.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          rb_, live ? (uint32_t)nl * 4 : dlane, 0, 0));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n0 + r < p.N ? n0 + r : (int)p.N - 1;
      const uint32_t off = live ? (uint32_t)((uint64_t)n * (uint64_t)p.ldq) + (uint32_t)s * 1024u + qlane
                                : dlane;
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq_, off, 0, 2));
      sl.q[r][0] = v.x; sl.q[r][1] = v.y; sl.q[r][2] = v.z; sl.q[r][3] = v.w;
    }
  };

  // A ring of D steps: while step t computes, the loads of steps t + 1 ..
  // t + D - 1 are in flight.
  StreamSlot<R> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    issue(j, ring[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // loads of a step: the scale (or per-channel scale), the bias, R rows; the
  // activation loads were issued before all of them, so they have landed once
  // no more than D steps' worth are outstanding
  constexpr int PER = 1 + (HASB ? 1 : 0) + R;
  asm volatile("" ::: "memory");
  wait_vmcnt<D * PER>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  float xr[32];
  auto load_x = [&](int s) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f4 t = *reinterpret_cast<const f4*>(xs + 4 * x_slot(s, lane, v));
      xr[4 * v + 0] = t.x; xr[4 * v + 1] = t.y; xr[4 * v + 2] = t.z; xr[4 * v + 3] = t.w;
    }
  };
  if (ONESPAN) load_x(0);
  const Magic mg = Magic::make();
  // integer products: the lane's chunk as digits, formed once
  uint32_t lim[7][4];
  float xe = 0.0f;
  if constexpr (IDOT) chunk_digits<ORDER>(xr, lim, xe);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  // rows n0, n0 + 1 leave once their last span is in: the 64-lane sums,
  // then lane r stores row n0 + r
  auto finish = [&](int n0, float e, float b) {
    float v = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sum = wave_sum(acc[r]);
      acc[r] = 0.0f;
      v = lane == r ? sum : v;
    }
    if (PERCH) v *= e;
    if (HASB) v += b;
    if (lane < R && n0 + lane < p.N) p.out[n0 + lane] = v;
  };

  // Whole rounds of D steps, every step issuing the loads of the step D
  // later (the same loads on every path keep the ring's registers in place
  // across iterations, so the compiler waits for each slot only where it is
  // used); steps past T compute nothing.
  int s = 0, i = 0;
  const int TR = (T + D - 1) / D * D;
  for (int t0 = 0; t0 < TR; t0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int t = t0 + j;
      const bool run = t < T;
      float e = 0.0f, b = 0.0f;
      bool last = false;
      int n0 = 0;
      if (run) {
        if (!ONESPAN) load_x(s);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float dot = IDOT ? chunk_dot_digits(ring[j].q[r], lim) * xe
                                 : chunk_dot<ORDER>(ring[j].q[r], xr, mg);
          acc[r] = PERCH ? acc[r] + dot : __builtin_fmaf(ring[j].s[r], dot, acc[r]);
        }
        e = ring[j].e;
        b = ring[j].b;
        last = s == S - 1;
        n0 = ((L + i * G) * W + wave) * R;
        if (++s == S) { s = 0; ++i; }
      }
      __builtin_amdgcn_sched_barrier(0);
      // the loads D steps ahead go out before this block's sums and store
      issue(t + D, ring[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (last) finish(n0, e, b);
    }
  }
}

template <int R, int ORDER, int SMODE, bool QA4, bool SA16, typename ST>
hipError_t launch_t(const GemvParams& p, dim3 grid, bool xl, hipStream_t s) {
  const int nwaves = p.waves_k * p.waves_r;
  if (xl)
    hipLaunchKernelGGL((gemv_f32_kernel<1, R, ORDER, SMODE, QA4, SA16, true, ST>), grid,
                       dim3(64 * nwaves), (size_t)p.waves_k * 8192, s, p);
  else
    hipLaunchKernelGGL((gemv_f32_kernel<1, R, ORDER, SMODE, QA4, SA16, false, ST>), grid,
                       dim3(64 * nwaves), 0, s, p);
  return hipGetLastError();
}

template <int R, int ORDER, int SMODE, bool SA16, int MB, typename ST>
hipError_t launch_lb_t(const GemvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemv_lb_kernel<R, ORDER, SMODE, SA16, MB, ST>), grid,
                     dim3(64 * p.waves_k * p.waves_r), (size_t)MB * p.waves_k * 8192, s, p);
  return hipGetLastError();
}

template <int R, int MB, typename ST>
hipError_t launch_lb_r(const GemvParams& p, dim3 grid, int order, int smode, bool sa16,
                       hipStream_t s) {
#define Q4_LB_CASE(O, S, B) \
  if (order == O && smode == S && sa16 == B) return launch_lb_t<R, O, S, B, MB, ST>(p, grid, s);
  Q4_LB_CASE(0, 0, false) Q4_LB_CASE(1, 0, false)
  Q4_LB_CASE(0, 1, false) Q4_LB_CASE(1, 1, false)
  Q4_LB_CASE(0, 1, true) Q4_LB_CASE(1, 1, true)
#undef Q4_LB_CASE
  return hipErrorInvalidValue;
}

template <int MB, typename ST>
hipError_t launch_lb(const GemvParams& p, dim3 grid, int R, int order, int smode, bool sa16,
                     hipStream_t s) {
  return R == 8   ? launch_lb_r<8, MB, ST>(p, grid, order, smode, sa16, s)
         : R == 4 ? launch_lb_r<4, MB, ST>(p, grid, order, smode, sa16, s)
                  : launch_lb_r<2, MB, ST>(p, grid, order, smode, sa16, s);
}

template <int R, typename ST>
hipError_t launch_r(const GemvParams& p, dim3 grid, bool xl, int order, int smode, bool qa4,
                    bool sa16, hipStream_t s) {
#define Q4_GEMV_CASE(O, S, A, B) \
  if (order == O && smode == S && qa4 == A && sa16 == B) return launch_t<R, O, S, A, B, ST>(p, grid, xl, s);
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


template <int W, int R, int ORDER, bool PERCH, int D, typename ST>
hipError_t launch_stream_d(const GemvParams& p, dim3 grid, hipStream_t s) {
  const size_t lds = (size_t)p.spans * 8192;
  const dim3 block(64 * W);
  if (p.spans == 1) {
    if (p.bias) hipLaunchKernelGGL((gemv_stream_kernel<W, R, ORDER, PERCH, true, true, D, ST, true>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((gemv_stream_kernel<W, R, ORDER, PERCH, true, false, D, ST, true>), grid, block, lds, s, p);
  } else {
    if (p.bias) hipLaunchKernelGGL((gemv_stream_kernel<W, R, ORDER, PERCH, false, true, D, ST>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((gemv_stream_kernel<W, R, ORDER, PERCH, false, false, D, ST>), grid, block, lds, s, p);
  }
  return hipGetLastError();
}

// the three shapes the plan uses: (waves, rows, depth) = (8, 2, 2), (4, 2, 2)
// and (4, 4, 1)
template <int ORDER, bool PERCH, typename ST>
hipError_t launch_stream_o(const GemvParams& p, const GemvLaunch& l, hipStream_t s) {
  if (l.R == 4) return launch_stream_d<4, 4, ORDER, PERCH, 1, ST>(p, l.grid, s);
  return l.waves == 8 ? launch_stream_d<8, 2, ORDER, PERCH, 2, ST>(p, l.grid, s)
                      : launch_stream_d<4, 2, ORDER, PERCH, 2, ST>(p, l.grid, s);
}

template <typename ST>
hipError_t launch_stream(const GemvParams& p, const GemvLaunch& l, hipStream_t s) {
  const bool perch = l.smode == kPerChannel;
  if (l.order == 0)
    return perch ? launch_stream_o<0, true, ST>(p, l, s) : launch_stream_o<0, false, ST>(p, l, s);
  return perch ? launch_stream_o<1, true, ST>(p, l, s) : launch_stream_o<1, false, ST>(p, l, s);
}

}  // namespace

template <typename ST>
hipError_t launch_gemv_kernels(const GemvParams& p, const GemvLaunch& l, hipStream_t s) {
  if (l.stream) return launch_stream<ST>(p, l, s);
  if (l.mb > 1)
    return l.mb == 8   ? launch_lb<8, ST>(p, l.grid, l.R, l.order, l.smode, l.sa16, s)
           : l.mb == 4 ? launch_lb<4, ST>(p, l.grid, l.R, l.order, l.smode, l.sa16, s)
                       : launch_lb<2, ST>(p, l.grid, l.R, l.order, l.smode, l.sa16, s);
  return l.R == 8   ? launch_r<8, ST>(p, l.grid, l.xl, l.order, l.smode, l.qa4, l.sa16, s)
         : l.R == 4 ? launch_r<4, ST>(p, l.grid, l.xl, l.order, l.smode, l.qa4, l.sa16, s)
                    : launch_r<2, ST>(p, l.grid, l.xl, l.order, l.smode, l.qa4, l.sa16, s);
}

}  // namespace q4
