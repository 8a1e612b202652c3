// q4_gemm.hip -- prefill GEMM for gfx950 (M > 1): binary16 operands on MFMA,
// fp32 accumulation.
//
// out[m, n] = sum_k RN16(x[m, k]) * RN16((q[n, k] - 8) * RN16(s[g(k), n]))
//             (+ bias[n]), summed in fp32.
// Precision recipe: binary16 operands, fp32 accumulator, never binary16
// accumulation (page 1, stack entry #20752: the binary16 multiply keeps an
// fp32 accumulator);
// every packed word and scale of a tile crosses into the chip once and is
// unpacked once (page 1, stack entry #20798, the packed-word-dequant
// staging).  The pages' 64x64 / 256-thread WGSL tile is prior art only.
//
// Layout on gfx950 (wave64, v_mfma_f32_32x32x16_f16, which sustains close to
// the dense binary16 peak where the 16x16x32 shape reaches about half):
//  * A pre-pass rounds the activations to binary16 once (RN16), in the k
//    order described below, zero-padded to whole tiles, into the workspace;
//    the GEMM then reads 2 bytes per activation instead of 4 on every
//    column tile that reuses it, and needs no row or K masks for them.
//  * Workgroups own 128 x 128 output tiles; K advances 64 per step.  The
//    pipelined kernel widens them to 128 x 256 where 128 x 128 tiles would
//    need more than one round of the 256 CUs and no split-K is planned:
//    each wave then owns 128 x 64 outputs, which halves the activation LDS
//    reads per MFMA (measured 9-11% faster on such shapes, slower where the
//    wider tiles leave CUs idle).
//  * Inside every 8-element group the k order follows the nibble order of
//    the packed word (pairs (i, i+4)); the activations are stored with the
//    same permutation, so A and B fragments pair up k for k.
//  * Two kernels.  The pipelined one (aligned rows, even K, power-of-two
//    groups >= 32 or per-channel scales) streams every operand into an LDS
//    ring with buffer loads that write LDS directly, and unpacks each weight
//    word once, in registers, into MFMA operands (details at the kernel);
//    when K is not a multiple of the 64-k step, the pre-pass also copies
//    each row's bytes of the last step (bytes past K as 0x88) and the
//    kernel reads that step from the copy.  The general one takes every
//    other shape: any group size, unaligned rows, odd K; it stages binary16
//    weight tiles in LDS from a register ring of global loads and masks the
//    edges (0x88 bytes past the end of a row, predicated stores).
//  * Scales come as fp32 or as binary16 (q4f16_1 weights); a binary16
//    scale is its own RN16, so both give the same operands.
//  * Split-K (grid.z > 1), only for deep K on few tiles, writes fp32
//    partials to the workspace; the shared reduce kernel sums them in split
//    order and adds the bias.
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

constexpr int KS = 64;          // k per pipeline step
constexpr int PITCH = KS + 8;   // LDS row pitch in halves
constexpr int BM = 128;         // output rows per workgroup
constexpr int DEPTH = 3;        // steps of global loads in flight (general kernel)

enum ScaleMode : int { kPerChannel = 0, kGroup32 = 1, kGroup8 = 2, kGeneric = 3 };

// Output tile of logical workgroup `tile` (after xcd_swizzle: consecutive
// logical ids share an XCD and its L2).  Tiles go in groups of up to
// kGroupM row tiles: inside a group the row tile varies fastest, then the
// column tile.  The 32 workgroups an XCD runs at once then cover at most 4
// row tiles x 8 column tiles, so each row tile's binary16 activations and
// each column tile's weights are fetched into that L2 a few times rather
// than once per workgroup (with the row tile fastest over all of M, as at
// M = 2048, every workgroup of an XCD read other activation rows).
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of(uint32_t tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  const uint32_t span = (uint32_t)kGroupM * (uint32_t)tiles_n;
  const uint32_t g = tile / span, r = tile - g * span;
  const int left = tiles_m - (int)g * kGroupM;
  const uint32_t gm = (uint32_t)(left < kGroupM ? left : kGroupM);
  tm = (int)(g * kGroupM + r % gm);
  tn = (int)(r / gm);
}

// x16[r * kp + k] = RN16(x[r, k']) for r < mp, k < kp, where inside each
// group of 8 the k' follow the nibble order of the packed words (pairs
// (i, i + 4)); rows >= M and k >= K are zero.  A thread converts 8
// elements; a workgroup covers 2048 k of a row, grid.y strides the rows.
// With qtail (K % 64 != 0, the pipelined kernel) the threads also copy, for
// every weight row n < N, the 32 bytes of its last 64-k step into qtail[n],
// bytes past the row's K / 2 replaced by 0x88 (codes 8, c = 0): the
// pipelined kernel reads that step from there, so no 16-byte piece of it
// extends past a row.
template <int ORDER>
__global__ void __launch_bounds__(256)
x16_kernel(const float* __restrict__ x, int64_t ldx, int64_t M, int64_t K,
           _Float16* __restrict__ x16, int64_t mp, int64_t kp,
           const uint8_t* __restrict__ qw, int64_t ldq, int64_t N,
           uint8_t* __restrict__ qtail) {
  if (qtail) {
    const int64_t kbyte = ((K - 1) / 64) * 32;  // first byte of the last step
    const int64_t rowb = K / 2;                  // bytes of a row (K even)
    const int64_t t = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nt = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t n = t; n < N; n += nt) {
      uint32_t w[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t o = kbyte + 4 * d + b;
          v |= (uint32_t)(o < rowb ? qw[n * ldq + o] : 0x88u) << (8 * b);
        }
        w[d] = v;
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(qtail + n * 32);
#pragma unroll
      for (int d = 0; d < 8; ++d) dst[d] = w[d];
    }
  }
  const int64_t k0 = (int64_t)blockIdx.x * 2048 + 8 * threadIdx.x;
  if (k0 >= kp) return;
  for (int64_t r = blockIdx.y; r < mp; r += gridDim.y) {
    const float* src = x + r * ldx + k0;
    float v[8];
    if (r < M && k0 + 8 <= K) {
      const f32x4_a4 a = *reinterpret_cast<const f32x4_a4*>(src);
      const f32x4_a4 b = *reinterpret_cast<const f32x4_a4*>(src + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (r < M && k0 + i < K) ? src[i] : 0.0f;
    }
    h8 h;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) h[sl] = (_Float16)v[pair_k<ORDER>(sl >> 1, sl & 1)];
    *reinterpret_cast<h8*>(x16 + r * kp + k0) = h;
  }
}

// BN = 128 or 256 output columns per workgroup; NT = 2 * BN threads: waves
// 2 (rows) x BN/64 (columns), each 64 x 64; thread t dequantizes half a
// step of column t / 2.
template <int BN, int ORDER, int SMODE, bool QA4>
struct Gemm {
  static constexpr int NT = 2 * BN;
  static constexpr int WAVES_N = BN / 64;
  static constexpr int WM = 64, WN = 64;  // per wave
  static constexpr int MI = 2, NI = 2;    // 32x32 blocks per wave
  static constexpr int AU = BM * KS / 8 / NT;  // 16-byte activation pieces per thread

  struct Stage {
    u32x4 a[AU];  // 16-byte pieces of the binary16 activation tile
    uint32_t q[4];
    float s[4];
  };

  const GemmParams& p;
  int tid, lane, wm, wn;
  int kz1;                  // end of this split's K range
  int row_bytes;
  int bcol;                 // this thread's weight column in the tile
  int bhalf;                // which 32-k half of each step it dequantizes
  bool nvalid;
  // streaming state, advanced by one step after every load
  const _Float16* pa[AU];   // the thread's activation pieces
  const uint8_t* pq;        // the thread's 16 packed bytes
  int64_t scol;             // scale column (n, or 0 past N)
  int kc;                   // first k of the thread's chunk
  h2 s16c;                  // per-channel scale, rounded once

  __device__ Gemm(const GemmParams& p_, int64_t m0, int64_t n0, int kz0, int kz1_)
      : p(p_), kz1(kz1_) {
    tid = threadIdx.x;
    lane = tid & 63;
    wm = (tid >> 6) / WAVES_N;
    wn = (tid >> 6) % WAVES_N;
    row_bytes = (int)((p.K + 1) >> 1);
    bcol = tid >> 1;
    bhalf = tid & 1;
    const int64_t ncol = n0 + bcol;
    nvalid = ncol < p.N;
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int unit = tid + u * NT;
      pa[u] = p.x16 + (m0 + (unit >> 3)) * p.x16_pitch + kz0 + 8 * (unit & 7);
    }
    kc = kz0 + 32 * bhalf;
    pq = p.qw + (nvalid ? ncol : 0) * p.ldq + (kc >> 1);
    scol = nvalid ? ncol : 0;
    if (SMODE == kPerChannel) s16c = splat_f16(nvalid ? scale(0) : 0.0f);
  }

  // scale of this thread's column in scale row g (fp32, or binary16 widened)
  __device__ __forceinline__ float scale(int64_t g) const {
    return scale_at(p.scales, p.scales16, g * p.lds + scol);
  }

  __device__ __forceinline__ int group_of(int k) const {
    return p.log2_gs >= 0 ? (k >> p.log2_gs) : k / (int)p.group_size;
  }

  template <bool GUARD>
  __device__ __forceinline__ void load(Stage& st) {
    // activations: already binary16, zero-padded to the tile grid
#pragma unroll
    for (int u = 0; u < AU; ++u) st.a[u] = *reinterpret_cast<const u32x4*>(pa[u]);
    const bool any = !GUARD || (nvalid && kc < kz1);
    const bool full = !GUARD || kc + 32 <= kz1;
    if (any) {
      if (full && QA4) {
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(pq);
        st.q[0] = v.x; st.q[1] = v.y; st.q[2] = v.z; st.q[3] = v.w;
      } else {
        const int byte0 = kc >> 1;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            // bytes past the row hold no k < K; their activations are 0
            const bool in = full || byte0 + 4 * d + b < row_bytes;
            w |= (in ? (uint32_t)pq[4 * d + b] : 0x88u) << (8 * b);
          }
          st.q[d] = w;
        }
      }
      if (SMODE == kGroup32) {
        st.s[0] = scale(group_of(kc));
      } else if (SMODE == kGroup8) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          int g = group_of(kc + 8 * d);
          g = g < (int)p.G - 1 ? g : (int)p.G - 1;
          st.s[d] = scale(g);
        }
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) { st.q[d] = 0x88888888u; st.s[d] = 0.0f; }
    }
#pragma unroll
    for (int u = 0; u < AU; ++u) pa[u] += KS;
    pq += KS / 2;
    kc += KS;
  }

  __device__ __forceinline__ void store(int kb, const Stage& st, _Float16* As,
                                        _Float16* Bs, const Magic& mg) const {
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int unit = tid + u * NT;
      const int r = unit >> 3, c = unit & 7;
      *reinterpret_cast<u32x4*>(&As[r * PITCH + 8 * c]) = st.a[u];
    }
    const int kcs = kb + 32 * bhalf;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      h2 c[4];
      unpack_word(st.q[d], mg, c);
      h2 w[4];
      if (SMODE == kGeneric) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            int g = (kcs + 8 * d + pair_k<ORDER>(pp, hh)) / (int)p.group_size;
            g = g < (int)p.G - 1 ? g : (int)p.G - 1;
            const _Float16 s16 = (_Float16)(nvalid ? scale(g) : 0.0f);
            const _Float16 cc = hh == 0 ? c[pp].x : c[pp].y;
            if (hh == 0) w[pp].x = cc * s16; else w[pp].y = cc * s16;
          }
      } else {
        const h2 s16 = SMODE == kPerChannel ? s16c
                       : SMODE == kGroup32  ? splat_f16(st.s[0])
                                            : splat_f16(st.s[d]);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) w[pp] = dequant_pair_f16(c[pp], s16);
      }
      const h8 hw = {w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
      *reinterpret_cast<h8*>(&Bs[bcol * PITCH + 32 * bhalf + 8 * d]) = hw;
    }
  }

  __device__ __forceinline__ void compute(const _Float16* As, const _Float16* Bs,
                                          f16v (&acc)[MI][NI]) const {
    const int li = lane & 31, lb = lane >> 5;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      h8 a[MI], b[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = *reinterpret_cast<const h8*>(&As[(wm * WM + i * 32 + li) * PITCH + 32 * lb + 8 * t]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        b[j] = *reinterpret_cast<const h8*>(&Bs[(wn * WN + j * 32 + li) * PITCH + 32 * lb + 8 * t]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <int BN, int ORDER, int SMODE, bool QA4>
__global__ void __launch_bounds__(2 * BN)
gemm_f16_kernel(const GemmParams p) {
  using G = Gemm<BN, ORDER, SMODE, QA4>;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * PITCH];

  const uint32_t tile = xcd_swizzle(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_of(tile, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int z = blockIdx.z;
  const int64_t kz0 = (int64_t)z * p.k_per_split;
  const int64_t kz1 = (kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K;
  const int nsteps = (int)((kz1 - kz0 + KS - 1) / KS);
  const bool inner_n = n0 + BN <= p.N;

  G g(p, m0, n0, (int)kz0, (int)kz1);
  const Magic mg = Magic::make();
  f16v acc[G::MI][G::NI];
#pragma unroll
  for (int i = 0; i < G::MI; ++i)
#pragma unroll
    for (int j = 0; j < G::NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Register ring of DEPTH staged steps: the global loads of step s+DEPTH
  // are issued while step s computes, so each load has DEPTH-1 steps of
  // MFMA work to arrive before its step is written to LDS.
  typename G::Stage st[DEPTH];
  // loads are issued in step order; g advances its pointers after each
  auto load_step = [&](int step, typename G::Stage& dst) {
    const int64_t kb = kz0 + (int64_t)step * KS;
    if (inner_n && kb + KS <= kz1) g.template load<false>(dst);
    else g.template load<true>(dst);
  };
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (i < nsteps) load_step(i, st[i]);
  if (nsteps > 0) g.store((int)kz0, st[0], As[0], Bs[0], mg);
  __syncthreads();
  for (int step0 = 0; step0 < nsteps; step0 += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int step = step0 + i;
      if (step < nsteps) {
        const int buf = step & 1;
        // slot i held this step; it is in LDS now, so it takes step + DEPTH
        if (step + DEPTH < nsteps) load_step(step + DEPTH, st[i]);
        g.compute(As[buf], Bs[buf], acc);
        if (step + 1 < nsteps)
          g.store((int)kz0 + (step + 1) * KS, st[(i + 1) % DEPTH], As[buf ^ 1], Bs[buf ^ 1],
                  mg);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: lane l, element v of a 32x32 block holds
  //      row 8*(v/4) + 4*(l/32) + v%4, column l%32 ----
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) / G::WAVES_N, wn = (threadIdx.x >> 6) % G::WAVES_N;
#pragma unroll
  for (int j = 0; j < G::NI; ++j) {
    const int64_t col = n0 + wn * G::WN + j * 32 + (lane & 31);
    if (col >= p.N) continue;
    const float bcol = (p.split == 1 && p.bias) ? p.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < G::MI; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * G::WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= p.M) continue;
        if (p.split > 1)
          p.partial[((int64_t)z * p.M + row) * p.N + col] = acc[i][j][v];
        else
          p.out[row * p.ldo + col] = acc[i][j][v] + bcol;
      }
  }
}

// Raw buffer resource over [base, base + bytes): reads past the end
// return 0.  bytes is clamped to the 32-bit record count.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// ---------------------------------------------------------------------------
// Pipelined fast path: power-of-two group sizes >= 32 or per-channel
// scales, even K, dword-aligned weight rows, every byte offset below 2^32;
// 128 x 128 tiles.  With K % 64 != 0 the last step's weights come from the
// pre-pass's 32-byte copy of each row (bytes past K as 0x88).
// Global memory reaches LDS by buffer loads that write LDS directly, so no
// registers hold data in flight and up to NSTAGE steps of activations,
// packed weights and scales are in flight at once: the workgroup waits for
// memory only when the pipeline runs dry.  Each of the 4 waves owns 32 output
// columns and all 128 rows (four 32x32 MFMA blocks that share one weight
// fragment), so every packed word is unpacked by exactly one lane, straight
// from LDS into the MFMA operand registers.
//
// k order inside a step of 64: MFMA t (0..3) takes k-chunks t (lanes 0-31)
// and 4 + t (lanes 32-63), chunk c = k 8c .. 8c+7 of the step.  A lane's
// four chunks 4*lb + t are then one 16-byte piece of its column's 32 packed
// bytes, and with 32-wide groups lane half lb lies in group 2*step + lb.
//
// LDS per stage: activations 128 rows x 8 chunks of 16 bytes, XOR-swizzled
// (a_slot); packed weights [128 NI columns][32 bytes]; scales
// [4 waves][NI blocks][2 halves][32 columns] floats.  Five stages: 105 KiB
// with NI = 1, 130 KiB with NI = 2.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Instruction order of one pipeline step, for the scheduler: a wave issues
// in order, and an MFMA keeps the matrix unit busy for 32 cycles, so each
// MFMA is followed by the next step's loads and LDS reads and by a few
// dequant VALU ops, which issue while it runs.
// NI: 32-column blocks per wave (16 NI MFMAs, 4 + 2 NI buffer loads and
// 1 + 16 + 2 NI LDS reads per step and wave).
template <int K, int NI>
__device__ __forceinline__ void interleave_slots() {
  if constexpr (K < 16 * NI) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (K < 4 + 2 * NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load
    if constexpr (K < 7 + 2 * NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
    if constexpr (K >= 4) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    interleave_slots<K + 1, NI>();
  }
}
template <int NI>
__device__ __forceinline__ void interleave_step() { interleave_slots<0, NI>(); }

// A wave-uniform pointer placed in scalar registers (a buffer resource must
// live in SGPRs; an address computed with 64-bit vector arithmetic would
// otherwise be re-checked lane by lane on every load).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// s_waitcnt with vmcnt(n) and lgkmcnt(0), expcnt left free (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

constexpr int PIPE_NT = 256;

// LDS slot (16 bytes) of activation chunk c (0..7) of tile row r.  Rows are
// 128 bytes; the XOR with bits 1..3 of the row puts the 16 rows that one
// 16-lane group of a ds_read_b128 touches on 16 distinct 4-bank groups.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// row pitch, in floats, of the output tile the epilogue stages in LDS
constexpr int EPI_TP = 136;

template <int NSTAGE, int NI>
struct PipeSmem {
  uint32_t a[NSTAGE][BM * KS / 2];          // binary16 activations, swizzled
  uint32_t q[NSTAGE][128 * NI * KS / 8];    // packed weights, 32 bytes per column
  float s[NSTAGE][PIPE_NT * NI];            // scales (grouped only)
};

// S16: binary16 scales (q4f16_1).  A lane's scale DMA then fetches the
// dword that holds its column's scale and its even/odd neighbour's (N and
// lds even, scales 4-byte aligned: no dword straddles the array's end) and
// keeps the half of its own column parity.
//
// NI: 32-column blocks per wave.  NI = 1: 128 x 128 tiles, a wave owns
// 128 x 32 outputs.  NI = 2: 128 x 256 tiles, a wave owns 128 x 64 (two
// column blocks sharing each activation fragment), which halves the
// activation LDS reads per MFMA; the per-output k order is the same.
template <int ORDER, bool PERCH, int NSTAGE, bool S16, int NI>
__global__ void __launch_bounds__(PIPE_NT)
gemm_pipe_kernel(const GemmParams p) {
  static_assert(NSTAGE >= 3 && NSTAGE <= 6, "pipeline depth");
  static_assert(NI == 1 || NI == 2, "column blocks per wave");
  constexpr int PER_STAGE = PERCH ? 4 + NI : 4 + 2 * NI;  // buffer loads per stage per lane
  static_assert(PER_STAGE * (NSTAGE - 1) < 64, "vmcnt range");
  static_assert(sizeof(PipeSmem<NSTAGE, NI>) >= BM * EPI_TP * sizeof(float),
                "the epilogue stages the output tile in the pipeline's LDS");
  static_assert(sizeof(PipeSmem<NSTAGE, NI>) <= 160 * 1024, "LDS per workgroup");
  // The kernel's only LDS object: with a second one the compiler can no
  // longer tell the loop's LDS reads from the LDS-DMA writes in flight and
  // waits for all of them (vmcnt(0)) before every step's reads, which drains
  // the ring (measured 35% slower).
  __shared__ __attribute__((aligned(16))) PipeSmem<NSTAGE, NI> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, in a scalar register: the LDS destination of a buffer load
  // (register M0) must be the same for the whole wave
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lb = lane >> 5;
  const uint32_t tile = xcd_swizzle(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_of(tile, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * (128 * NI);
  const int c0 = 32 * NI * w;  // first tile column of this wave
  const int z = blockIdx.z;
  const int kz0 = (int)((int64_t)z * p.k_per_split);
  const int kz1 = (int)((kz0 + p.k_per_split < p.K) ? kz0 + p.k_per_split : p.K);
  const int nsteps = (kz1 - kz0 + KS - 1) / KS;

  // Buffer resources over the exact extents the caller guarantees; every
  // read past them returns 0 (the range check covers the per-lane offset,
  // which therefore carries the step's k).
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(uniform_ptr(p.x16 + m0 * p.x16_pitch), (uint64_t)BM * p.x16_pitch * 2);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(p.qw, (uint64_t)(p.N - 1) * p.ldq + (uint64_t)((p.K + 1) >> 1));
  // the last 64-k step's weights from the pre-pass's copy when K % 64 != 0
  // (kb_tail never matches a step otherwise)
  const __amdgpu_buffer_rsrc_t rqt = make_rsrc(p.qtail, p.qtail ? (uint64_t)p.N * 32 : 0);
  const uint32_t kb_tail = p.qtail ? (uint32_t)(((p.K - 1) / KS) * KS) : 0xFFFFFFFFu;
  constexpr uint32_t SB = S16 ? 2 : 4;  // bytes per scale
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(S16 ? (const void*)p.scales16 : (const void*)p.scales,
                ((uint64_t)(p.G - 1) * p.lds + (uint64_t)p.N) * SB);

  // this lane's activation slots: wave w fills slots 256w .. 256w + 255
  uint32_t va[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = (w * 4 + u) * 64 + lane;  // slot j = a_slot(row, c)
    const int row = j >> 3, c = (j & 7) ^ ((row >> 1) & 7);
    va[u] = (uint32_t)((row * p.x16_pitch + 8 * c) * 2);
  }
  // packed weights of column block u: lane -> column c0 + 32u + lane/2,
  // 16-byte half lane & 1.  The arrays have a fixed bound (NI <= 2): with a
  // bound taken from the template arguments, the lambda below that captures
  // them leaves the kernel without its host-side launch stub.
  uint32_t vq[2], vs[2], vt[2];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    vq[u] = (uint32_t)((n0 + c0 + 32 * u + (lane >> 1)) * p.ldq + 16 * (lane & 1));
    vt[u] = (uint32_t)((n0 + c0 + 32 * u + (lane >> 1)) * 32 + 16 * (lane & 1));
    // scales of block u: lane -> half lb's group, column c0 + 32u + li
    vs[u] = (uint32_t)(((n0 + c0 + 32 * u + li) & (S16 ? ~1 : ~0)) * SB);
  }
  const uint32_t lds4 = (uint32_t)(p.lds * SB);
  const int l2g = p.log2_gs;

  auto issue = [&](int st, int step) {
    const uint32_t kb = (uint32_t)(kz0 + step * KS);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_ptr_t)((char*)&sm.a[st][0] + (w * 4 + u) * 1024), 16, va[u] + 2 * kb, 0, 0, 0);
    const bool tail = kb == kb_tail;
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          tail ? rqt : rq, (lds_ptr_t)((char*)&sm.q[st][0] + (w * NI + u) * 1024), 16,
          tail ? vt[u] : vq[u] + (kb >> 1), 0, 0, 0);
    if (!PERCH)
#pragma unroll
      for (int u = 0; u < NI; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_ptr_t)((char*)&sm.s[st][0] + (w * NI + u) * 256), 4,
            vs[u] + ((kb + 32 * lb) >> l2g) * lds4, 0, 0, 0);
  };

  h2 s16c[2];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    s16c[u] = h2{(_Float16)0.0f, (_Float16)0.0f};
    if (PERCH) {
      const int64_t col = n0 + c0 + 32 * u + li;
      s16c[u] = splat_f16(col < p.N ? scale_at(p.scales, p.scales16, col) : 0.0f);
    }
  }
  const Magic mg = Magic::make();

  f16v acc[NI][4];
#pragma unroll
  for (int u = 0; u < NI; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[u][i][v] = 0.0f;

  // A step's operands, read from LDS into registers one step ahead, and its
  // weights dequantized one step ahead: while the MFMAs of step s run, the
  // wave issues the LDS reads of step s + 1 and unpacks its weights.
  struct Frag {
    h8 a[4][4];   // [t][i]: activation rows 32i + li, chunk 4 lb + t
    h8 b[NI][4];  // [u][t]: binary16 weights of this lane's column in block u, chunk 4 lb + t
    u32x4 q[NI];  // packed words of those columns, chunks 4 lb .. 4 lb + 3
    float s[NI];  // their scales for this lane's half-step (grouped)
  };
  auto read_frag = [&](int st, Frag& f) {
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      f.q[u] = *reinterpret_cast<const u32x4*>((const char*)&sm.q[st][0] + (w * NI + u) * 1024 +
                                               li * 32 + lb * 16);
      if (!PERCH && !S16) f.s[u] = sm.s[st][(w * NI + u) * 64 + lane];
      if (!PERCH && S16) {
        const uint32_t d = __builtin_bit_cast(uint32_t, sm.s[st][(w * NI + u) * 64 + lane]);
        f.s[u] = (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> (16 * (li & 1))));
      }
    }
    const char* abase = (const char*)&sm.a[st][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f.a[t][i] = *reinterpret_cast<const h8*>(abase + a_slot(i * 32 + li, 4 * lb + t) * 16);
  };
  auto dequant = [&](Frag& f) {
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const h2 s16 = PERCH ? s16c[u] : splat_f16(f.s[u]);
      const uint32_t qw4[4] = {f.q[u].x, f.q[u].y, f.q[u].z, f.q[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h2 c[4];
        unpack_word(qw4[t], mg, c);
        h2 d[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) d[pp] = dequant_pair_f16(c[pp], s16);
        f.b[u][t] = h8{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
      }
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[u][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[t][i], f.b[u][t], acc[u][i], 0, 0, 0);
  };

  // Pipeline.  The prologue puts steps 0 .. NSTAGE-1 in flight (one per
  // stage) and reads step 0 into registers.  Iteration s waits for its own
  // loads of step s + 1 (the NSTAGE-2 younger steps may still be in flight)
  // and for its LDS reads of step s, then meets the other waves: their loads
  // of step s + 1 have landed and their reads of step s are done, so step
  // s's stage is refilled with step s + NSTAGE.  It then issues the LDS reads
  // of step s + 1 and runs the MFMAs of step s.  Loads past the last step
  // read zeros or unused bytes, are never computed, and are drained before
  // the epilogue.
  constexpr int UNROLL = (NSTAGE % 2 == 0) ? NSTAGE : 2 * NSTAGE;
  Frag fa, fb;
  wait_vm_lgkm0<0>();
#pragma unroll
  for (int st = 0; st < NSTAGE; ++st) issue(st, st);
  wait_vm_lgkm0<PER_STAGE * (NSTAGE - 1)>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frag(0, fa);
  dequant(fa);
  for (int s0 = 0; s0 < nsteps; s0 += UNROLL) {
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      if (s0 + j < nsteps) {
        Frag& cur = (j % 2 == 0) ? fa : fb;
        Frag& nxt = (j % 2 == 0) ? fb : fa;
        wait_vm_lgkm0<PER_STAGE * (NSTAGE - 2)>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(j % NSTAGE, s0 + j + NSTAGE);
        read_frag((j + 1) % NSTAGE, nxt);
        mma(cur);
        dequant(nxt);
        interleave_step<NI>();
      }
    }
  }
  wait_vm_lgkm0<0>();

  // Epilogue.  Every wave's loads have landed and its LDS reads are done, so
  // the ring is free: the tile goes through LDS and leaves as 16-byte
  // row-contiguous stores (with NI = 1 a wave writes two 512-byte row
  // segments per store; with NI = 2, eight 128-byte ones), non-temporal for
  // the output, which nothing here reads again.
  // The output write is the one serial phase after the MFMA loop: with
  // 4-byte stores straight from the MFMA layout (two 128-byte segments per
  // store) it took about 7.5 us of a 34 us call at M = 512, N = 8192; staged
  // like this, about 1.6 us.
  // Lane l, element v of a 32x32 block holds row 8*(v/4) + 4*(l/32) + v%4
  // and column l%32; the row pitch (EPI_TP floats) puts the two row halves
  // of one LDS store on disjoint banks.  With NI = 2 the tile leaves in two
  // passes, column block h of every wave in pass h.
  float* dst0;
  int64_t pitch;
  bool vec;
  if (p.split > 1) {
    dst0 = p.partial + (int64_t)z * p.M * p.N;
    pitch = p.N;
    vec = p.N % 4 == 0 && reinterpret_cast<uintptr_t>(dst0) % 16 == 0;
  } else {
    dst0 = p.out;
    pitch = p.ldo;
    vec = p.ldo % 4 == 0 && reinterpret_cast<uintptr_t>(p.out) % 16 == 0;
  }
  const bool addb = p.split == 1 && p.bias;
  float* ctile = reinterpret_cast<float*>(&sm);
  const int c4 = tid & 31;  // column quad of the staged 128 columns
#pragma unroll
  for (int h = 0; h < NI; ++h) {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        ctile[(i * 32 + 8 * (v >> 2) + 4 * lb + (v & 3)) * EPI_TP + 32 * w + li] = acc[h][i][v];
    __syncthreads();
    // staged column 4 c4 is column 4 (c4 % 8) of block h of wave c4 / 8
    const int64_t col = n0 + 32 * NI * (c4 >> 3) + 32 * h + 4 * (c4 & 7);
    f4 bq = {0.0f, 0.0f, 0.0f, 0.0f};
    if (addb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bq[e] = col + e < p.N ? p.bias[col + e] : 0.0f;
    }
#pragma unroll 4
    for (int j = 0; j < BM / 8; ++j) {
      const int r = (tid >> 5) + 8 * j;
      const int64_t row = m0 + r;
      if (row >= p.M) break;
      f4 v = *reinterpret_cast<const f4*>(ctile + r * EPI_TP + 4 * c4);
      if (addb) v += bq;
      float* dst = dst0 + row * pitch + col;
      if (vec && col + 4 <= p.N) {
        if (p.split > 1)
          *reinterpret_cast<f4*>(dst) = v;
        else
          __builtin_nontemporal_store(v, reinterpret_cast<f4*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < p.N) dst[e] = v[e];
      }
    }
  }
}

template <int ORDER, bool PERCH, bool S16>
hipError_t launch_pipe_t(const GemmParams& p, dim3 grid, bool wide, hipStream_t s) {
  if (wide)
    hipLaunchKernelGGL((gemm_pipe_kernel<ORDER, PERCH, 5, S16, 2>), grid, dim3(PIPE_NT), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_pipe_kernel<ORDER, PERCH, 5, S16, 1>), grid, dim3(PIPE_NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pipe(const GemmParams& p, dim3 grid, int order, bool perch, bool wide,
                       hipStream_t s) {
  // per-channel scales are read once per lane, outside the pipeline
  const bool s16 = p.scales16 != nullptr && !perch;
  if (order == 0) {
    if (perch) return launch_pipe_t<0, true, false>(p, grid, wide, s);
    return s16 ? launch_pipe_t<0, false, true>(p, grid, wide, s)
               : launch_pipe_t<0, false, false>(p, grid, wide, s);
  }
  if (perch) return launch_pipe_t<1, true, false>(p, grid, wide, s);
  return s16 ? launch_pipe_t<1, false, true>(p, grid, wide, s)
             : launch_pipe_t<1, false, false>(p, grid, wide, s);
}

// 128 x 256 tiles for the pipelined kernel: only without split-K, and only
// where 128 x 128 tiles would take more than one round of the chip's 256
// CUs (then the wider tiles' cheaper steps outweigh the lost parallelism).
bool pipe_wide(const GemmPlan& pl) {
  return pl.split == 1 && (int64_t)pl.tiles_m * pl.tiles_n > 256;
}

template <int BN, int ORDER, int SMODE, bool QA4>
hipError_t launch_t(const GemmParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f16_kernel<BN, ORDER, SMODE, QA4>), grid, dim3(2 * BN), 0, s, p);
  return hipGetLastError();
}

template <int BN>
hipError_t launch_cfg(const GemmParams& p, dim3 grid, int order, int smode, bool qa4,
                      hipStream_t s) {
#define Q4_GEMM_CASE(O, S, A) \
  if (order == O && smode == S && qa4 == A) return launch_t<BN, O, S, A>(p, grid, s);
  Q4_GEMM_CASE(0, 0, true) Q4_GEMM_CASE(0, 1, true) Q4_GEMM_CASE(0, 2, true) Q4_GEMM_CASE(0, 3, true)
  Q4_GEMM_CASE(1, 0, true) Q4_GEMM_CASE(1, 1, true) Q4_GEMM_CASE(1, 2, true) Q4_GEMM_CASE(1, 3, true)
  Q4_GEMM_CASE(0, 0, false) Q4_GEMM_CASE(0, 1, false) Q4_GEMM_CASE(0, 2, false) Q4_GEMM_CASE(0, 3, false)
  Q4_GEMM_CASE(1, 0, false) Q4_GEMM_CASE(1, 1, false) Q4_GEMM_CASE(1, 2, false) Q4_GEMM_CASE(1, 3, false)
#undef Q4_GEMM_CASE
  return hipErrorInvalidValue;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  (void)group_size;
  GemmPlan pl{};
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t ksteps = (K + KS - 1) / KS;
  // 128 x 128 output tiles
  pl.cfg = 128;
  pl.tiles_m = (int)tiles_m;
  pl.tiles_n = (int)((N + pl.cfg - 1) / pl.cfg);
  const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
  // Split K where the tiles alone leave CUs idle, down to 8 steps per split:
  // each split adds an fp32 write and read of the output, small next to the
  // weights when the tiles are few (small M or narrow N).
  int split = 1;
  while (tiles * split * 2 <= 256 && ksteps / (split * 2) >= 8) split *= 2;
  pl.k_per_split = ((ksteps + split - 1) / split) * KS;
  pl.split = (int)((K + pl.k_per_split - 1) / pl.k_per_split);
  pl.x16_rows = tiles_m * BM;
  pl.x16_pitch = ksteps * KS;
  return pl;
}

// workspace: [binary16 activations x16 | split-K partials] for the tiled
// kernel; the skinny kernel's split-K partials where it applies.  The query
// knows the sizes only (not the pointers that decide between the two), so it
// asks for the larger.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  const GemmPlan pl = plan_gemm(M, N, K, group_size);
  size_t b = align256((size_t)pl.x16_rows * (size_t)pl.x16_pitch * sizeof(_Float16));
  if (pl.split > 1) b += align256((size_t)pl.split * (size_t)M * (size_t)N * sizeof(float));
  if (K % KS != 0) b += (size_t)N * 32;  // the last step's weights (pipelined kernel)
  const size_t sk = skinny_workspace_bytes(M, N, K, group_size);
  return b > sk ? b : sk;
}

hipError_t launch_gemm(const GemmParams& p0, int order, bool qa4, void* workspace,
                       hipStream_t s, bool* skinny) {
  const SkinnyPlan sp = plan_skinny(p0.M, p0.N, p0.K, p0.group_size);
  const bool sk = skinny_fits(p0, sp, qa4);
  if (skinny) *skinny = sk;
  if (sk) return launch_skinny(p0, sp, order, workspace, s);
  GemmParams p = p0;
  const GemmPlan pl = plan_gemm(p.M, p.N, p.K, p.group_size);
  p.split = pl.split;
  p.k_per_split = pl.k_per_split;
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.x16_pitch = pl.x16_pitch;
  char* ws = reinterpret_cast<char*>(workspace);
  p.x16 = reinterpret_cast<_Float16*>(ws);
  const size_t x16_bytes = align256((size_t)pl.x16_rows * (size_t)pl.x16_pitch * sizeof(_Float16));
  p.partial = reinterpret_cast<float*>(ws + x16_bytes);
  p.qtail = nullptr;
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
  p.log2_gs = -1;  // group index by shift when the group size is a power of two
  if (smode != kPerChannel && (p.group_size & (p.group_size - 1)) == 0) {
    int l2 = 0;
    while ((1LL << l2) < p.group_size) ++l2;
    p.log2_gs = l2;
  }
  // The branch-free kernel: power-of-two groups >= 32 or per-channel,
  // dword-aligned rows, even K, and all byte offsets of its buffers below
  // 2^32.  Every 16-byte weight piece of its steps lies inside a row except
  // in the last 64-k step when K % 64 != 0 (a vector load that crosses the
  // end of its resource returns zeros for all of its bytes, and one inside
  // another row's bytes would bring codes that need not be 8): that step is
  // read from the pre-pass's copy, whose bytes past K are 0x88.
  const bool pow2 = smode == kGroup32 && p.log2_gs >= 5;
  const bool small = (uint64_t)p.N * (uint64_t)p.ldq < (1ull << 32) &&
                     (uint64_t)p.G * (uint64_t)p.lds * 4 < (1ull << 32) &&
                     (uint64_t)pl.x16_rows * (uint64_t)pl.x16_pitch * 2 < (1ull << 32);
  // binary16 grouped scales are fetched a dword (two columns) at a time:
  // N and lds even and the array 4-byte aligned
  const bool s16ok = !p.scales16 || smode == kPerChannel ||
                     (p.N % 2 == 0 && p.lds % 2 == 0 &&
                      reinterpret_cast<uintptr_t>(p.scales16) % 4 == 0);
  const bool pipe = qa4 && small && s16ok && p.K % 2 == 0 && (smode == kPerChannel || pow2);
  if (pipe && p.K % KS != 0)
    p.qtail = reinterpret_cast<uint8_t*>(ws) + x16_bytes +
              (pl.split > 1 ? align256((size_t)pl.split * (size_t)p.M * (size_t)p.N * sizeof(float))
                            : 0);
  // 1. activations to binary16 (RN16), permuted and zero-padded; the last
  // step's weights for the pipelined kernel when K % 64 != 0
  const dim3 xgrid((unsigned)((pl.x16_pitch + 2047) / 2048),
                   (unsigned)(pl.x16_rows < 65535 ? pl.x16_rows : 65535));
  if (order == 0)
    hipLaunchKernelGGL(x16_kernel<0>, xgrid, dim3(256), 0, s, p.x, p.ldx, p.M, p.K, p.x16,
                       pl.x16_rows, pl.x16_pitch, p.qw, p.ldq, p.N, p.qtail);
  else
    hipLaunchKernelGGL(x16_kernel<1>, xgrid, dim3(256), 0, s, p.x, p.ldx, p.M, p.K, p.x16,
                       pl.x16_rows, pl.x16_pitch, p.qw, p.ldq, p.N, p.qtail);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. the GEMM
  if (pipe) {
    const bool wide = pipe_wide(pl);
    if (wide) p.tiles_n = (int)((p.N + 255) / 256);
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n), 1, (unsigned)pl.split);
    e = launch_pipe(p, grid, order, smode == kPerChannel, wide, s);
  } else {
    const dim3 grid((unsigned)(pl.tiles_m * pl.tiles_n), 1, (unsigned)pl.split);
    e = launch_cfg<128>(p, grid, order, smode, qa4, s);
  }
  if (e != hipSuccess || pl.split == 1) return e;
  // 3. split-K partial sums, in split order
  return launch_splitk_reduce(p.partial, p.bias, p.out, p.ldo, p.M, p.N, p.split, s);
}

}  // namespace q4
