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
//    rows of the workgroup, one 16-byte load per four rows (8 bytes when
//    the scales are binary16, q4f16_1 weights: widened exactly to fp32).
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
//  * Deep K (four or more spans) and very large single-span shapes run a
//    second, streaming kernel instead (gemv_stream_kernel): each workgroup
//    stages the activations once and its waves loop over row blocks, every
//    wave covering all of K for its rows, with the next step's loads in
//    flight while one computes.  No span waves meet in LDS and no split-K
//    reduce runs for K <= 16384.  With one span (the output head) a lane's
//    activation chunk serves every row its wave visits, so that kernel
//    rewrites it once as block fixed point (27 bits against the chunk's
//    largest |x|) and forms the products exactly with 4-bit integer dot
//    products (q4_gemv_kernels.h describes the arithmetic).
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

using namespace gemv;

int scale_mode(int64_t gs, int64_t K) {
  if (gs == 0 || gs >= K) return kPerChannel;
  const bool pow2 = (gs & (gs - 1)) == 0;
  if (pow2 && gs >= 32 && gs <= 2048) return kStaged;
  return kGeneric;
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

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  (void)group_size;
  GemvPlan pl{};
  pl.cfg = 1;  // one chunk of 32 k per lane; a wave spans 2048 k
  const int64_t spans = (K + 2047) / 2048;
  pl.split = (int)((spans + 7) / 8);  // at most 8 span-waves per workgroup
  pl.waves_k = (int)((spans + pl.split - 1) / pl.split);
  pl.k_per_split = (int64_t)pl.waves_k * 2048;
  // More than two activation rows want the low-batch kernel to hold them in
  // one workgroup, whose LDS takes at most 8 / waves_k of them: with four
  // span waves the weights would stream once per two rows.  K is then split
  // in two, so two spans meet per workgroup and it holds four rows, for the
  // cost of the reduce launch (measured on MI355X for 8192 x 2048 at M = 4:
  // 15.8 -> 13.3 us; at M = 16: 54.5 -> 37.1 us).  Deeper K is left as it
  // is: splitting 14336 x 4096 in four was slower at M = 3 and 4.
  if (M > 2 && pl.split == 1 && pl.waves_k == 4) {
    pl.split = 2;
    pl.waves_k = 2;
    pl.k_per_split = 4096;
  }
  // Rows per wave and row groups per workgroup, from a sweep on MI355X over
  // the Llama-shaped projections: about four waves per workgroup, four rows
  // per wave unless that leaves fewer than 2048 waves (then two), eight
  // only for deep K (more than four spans) where eight still give 2048;
  // for one activation row, two spans over at most 4096 rows run two rows
  // per wave in four row groups, and four spans two row groups (eight waves
  // sharing the activations).
  pl.mb = lowbatch_rows(M, pl.waves_k);
  const int64_t mrows = (M + pl.mb - 1) / pl.mb;  // activation row blocks
  auto waves = [&](int r) { return ((N + r - 1) / r) * pl.waves_k * pl.split * mrows; };
  int rows = 4;
  if (waves(4) < 2048) rows = 2;
  if (pl.waves_k > 4 && waves(8) >= 2048) rows = 8;
  int wr = 4 / pl.waves_k;
  if (pl.mb == 1 && mrows == 1 && pl.waves_k == 2 && N <= 4096) { rows = 2; wr = 4; }
  if (pl.mb == 1 && mrows == 1 && pl.waves_k == 4) wr = 2;
  pl.rows_per_wave = rows;
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

// The streaming kernel's domain: one activation row; K a multiple of 32
// (every 16-byte chunk of a row lies inside the row or wholly past its
// end) and at most 8 spans of 2048 (the activations fit its LDS);
// dword-aligned weight rows; power-of-two groups of 32 .. 2048 or
// per-channel scales, binary16 pairs dword-aligned; every byte offset
// below 2^32 (its buffer resources).  Other one-row shapes run
// gemv_f32_kernel.
static bool use_stream(const GemvParams& p, int smode, bool qa4) {
  if (p.M != 1 || !qa4 || p.K % 32 != 0 || p.K > 8 * 2048) return false;
  // where it measured faster than gemv_f32_kernel on MI355X: deep K (four
  // or more spans: no span waves meeting in LDS) or very many weights (the
  // 2048 x 128257 output head); at the 1B projections' other sizes the
  // one-pass kernel, whose every load is in flight from the start, is faster
  if (!(p.K >= 4 * 2048 || (double)p.N * (double)p.K >= (double)(1 << 27))) return false;
  if (smode != kStaged && smode != kPerChannel) return false;
  if (p.scales16 && smode == kStaged &&
      (p.lds % 2 != 0 || reinterpret_cast<uintptr_t>(p.scales16) % 4 != 0))
    return false;
  const uint64_t sb = p.scales16 ? 2 : 4;
  const uint64_t scale_bytes =
      smode == kPerChannel ? (uint64_t)p.N * sb : ((uint64_t)(p.G - 1) * p.lds + p.N) * sb;
  return (uint64_t)p.N * (uint64_t)p.ldq < (1ull << 32) && scale_bytes < (1ull << 32) &&
         (uint64_t)p.N * 4 < (1ull << 31);
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
  const bool sa16 = smode == kStaged && R >= 4 && (p.lds % 4 == 0) &&
                    (p.scales16 ? reinterpret_cast<uintptr_t>(p.scales16) % 8 == 0
                                : reinterpret_cast<uintptr_t>(p.scales) % 16 == 0);
  p.rows_per_block = (int32_t)rpb;
  // several activation rows per workgroup (weights read once for all):
  // aligned weights, activations through LDS, staged or per-channel scales
  const int mb = (xl && qa4 && smode != kGeneric) ? pl.mb : 1;
  GemvLaunch l{};
  l.grid = dim3((unsigned)((p.N + rpb - 1) / rpb), (unsigned)((p.M + mb - 1) / mb),
                (unsigned)pl.split);
  l.R = R; l.mb = mb; l.xl = xl; l.order = order; l.smode = smode; l.qa4 = qa4; l.sa16 = sa16;
  if (use_stream(p, smode, qa4)) {
    // one activation row on aligned shapes: the streaming kernel (no split)
    // One span over very many rows (the output head): four rows per wave
    // step, four waves, one step in flight.  Deep K: two rows per step and
    // two steps in flight, eight waves per workgroup, four when eight would
    // leave CUs without a block (N < 4096).  Measured on MI355X against the
    // other (waves, rows, depth) combinations on the Llama-shaped shapes.
    const bool head = p.K <= 2048;
    l.R = head ? 4 : 2;
    l.waves = head || p.N < 4096 ? 4 : 8;
    l.depth = head ? 1 : 2;
    const int rows = l.waves * l.R;
    p.spans = (int32_t)((p.K + 2047) / 2048);
    p.blocks = (int32_t)((p.N + rows - 1) / rows);
    p.split = 1;
    l.stream = true;
    l.grid = dim3((unsigned)(p.blocks < kStreamMaxGrid ? p.blocks : kStreamMaxGrid));
    return p.scales16 ? launch_gemv_kernels<_Float16>(p, l, s) : launch_gemv_kernels<float>(p, l, s);
  }
  const hipError_t e = p.scales16 ? launch_gemv_kernels<_Float16>(p, l, s)
                                  : launch_gemv_kernels<float>(p, l, s);
  if (e != hipSuccess || pl.split == 1) return e;
  return launch_splitk_reduce(p.partial, p.bias, p.out, p.ldo, p.M, p.N, p.split, s);
}

}  // namespace q4
