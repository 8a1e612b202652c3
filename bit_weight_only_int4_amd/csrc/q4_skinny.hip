// q4_skinny.hip -- the plan of the few-row MFMA GEMM (1 <= M <= 1024) and its
// launch; the kernel and its design are in q4_skinny_kernels.h.
#include "q4_kernels.h"

namespace q4 {
namespace {
constexpr int SK_W = 8;       // waves per workgroup (as in the kernel)
constexpr int SK_STEP = 128;  // k per wave step
}  // namespace

// LDS for the activations of one slice (M rows x k_slice binary16) plus,
// with waves split along K, the partial sums (8 waves x 8 or 16 floats per
// lane).  One row of the plan per call, from the sizes alone.
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t group_size) {
  SkinnyPlan pl{};
  const bool perch = group_size == 0 || group_size >= K;
  const bool pow2 = group_size >= 32 && (group_size & (group_size - 1)) == 0;
  // Above 32 rows (row blocks of 32, each reading the weights) the kernel is
  // taken where it was measured faster than the tiled GEMM on MI355X: at
  // M = 64 on the Llama-3.2-1B projections (N * K <= 2^24: 11.0-17.4 us
  // against 13.7-21.9), the 8B q projection (16.3 against 20.4) and the
  // vocabulary-sized output head (71.6 against 83.5), not on the 8B gate/up
  // and down projections (31.4 and 32.4 against 27.9 and 29.4); and on
  // narrow N (<= 4096) with N * K <= 2^24, where the tiled GEMM has few
  // tiles and splits K, up to 1024 rows while M * N * K <= 2^31 (larger
  // weights lost even at 33-40 rows: 14336 x 4096 31.4-32.0 against
  // 27.7-28.4 us, 12288 x 4096 29.0 against 26.4): e.g. K x N = 2048 x 2048 at
  // M = 65-128 9.4-10.1 against 14.7-16.4 us, at 256 12.8 against 19.7, at
  // 512 19.2 against 23.7; 8192 x 2048 at M = 97-128 22.2-23.0 against
  // 23.4-26.1; 2008 x 3000 at 65-320 11.8-16.9 against 17.3-24.7; 1024 x
  // 1024 at 1024 13.3 against 20.3.  Beyond it the few-row kernel lost
  // (8192 x 2048 at 160-256: 28.9-39.3 against 24.4-26.6; 2048 x 2048 at
  // 768: 29.4 against 26.1), as it did on 2048 x 8192 at M = 65-96 (17.7-18.2
  // against 15.9-17.4).  Inside, the one loss measured: 2048 x 1024 at
  // M = 1024, 23.3 against 22.5.
  const double nk = (double)N * (double)K;
  const bool rows_ok = M <= 32 || (M <= 64 && (nk <= (double)(1LL << 25) || N >= 65536)) ||
                       (M <= 1024 && N <= 4096 && nk <= (double)(1LL << 24) &&
                        (double)M * nk <= (double)(1LL << 31));
  // K: whole 8-k chunks (K % 8 == 0).  The weight bytes past K of the
  // 32-k chunk that straddles K meet zero activations as exact codes where
  // the scale is taken out of the sums (per-channel, groups >= 128), and get
  // a zero scale otherwise (see the kernel)
  const bool kok = K % 8 == 0;
  pl.ok = M >= 1 && rows_ok && N >= 1 && K >= SK_STEP && kok && (perch || pow2) &&
          K <= ((int64_t)1 << 24);
  if (!pl.ok) return pl;
  // more than 32 rows: row blocks of 32 in separate workgroups
  pl.mz = (int)((M + 31) / 32);
  pl.mrows = pl.mz == 1 ? (int)M : 32;
  pl.mb = pl.mrows <= 16 ? 1 : 2;
  pl.ni = 2;
  const int64_t red = (int64_t)SK_W * pl.ni * pl.mb * 4 * 64 * 4;  // bytes
  constexpr int64_t kLds = 160 * 1024;
  const int64_t steps = (K + SK_STEP - 1) / SK_STEP;
  const int64_t per_step = (int64_t)SK_STEP * pl.mrows * 2;
  const int64_t max_steps = (kLds - red) / per_step;
  int64_t split = (steps + max_steps - 1) / max_steps;
  const int64_t sps = (steps + split - 1) / split;
  split = (steps + sps - 1) / sps;
  pl.split = (int)split;
  pl.k_slice = sps * SK_STEP;
  // waves along K: as few as leave at least 256 workgroup column blocks
  const int64_t ncb = (N + 16 * pl.ni - 1) / (16 * pl.ni);  // a wave's column blocks
  int wk = 8;
  for (int c = 1; c <= 8; c *= 2)
    if ((ncb * c + 7) / 8 >= 256) { wk = c; break; }
  while (wk > 1 && wk > sps) wk /= 2;
  const int64_t blocks = (ncb + SK_W / wk - 1) / (SK_W / wk);
  // Narrow N over deep K (the down projections at few rows) leaves CUs
  // without a block even with all 8 waves along K: split K further, while
  // every wave keeps at least two steps.  The partial sums (M x N floats
  // per split) are small next to the weights at these row counts.  Taken
  // where it measured faster on MI355X: waves with at least 8 steps (1B
  // down at M <= 16: 11.6-14.9 -> 9.7-11.2 us; 8B down at M <= 4: 16.4-18.3
  // -> 14.3-15.2 us) or at least 16 rows (8B q at M = 16: 11.1 -> 9.9 us);
  // with 4 steps per wave and fewer rows the reduce launch costs more than
  // the parallelism gains (8B q at M <= 8: +0.4-0.9 us).
  const bool deep = (sps + wk - 1) / wk >= 8 || pl.mrows >= 16;
  int64_t sps2 = sps, split2 = split;
  while (deep && blocks * split2 * pl.mz < 256 && sps2 >= 4 * wk) {
    split2 *= 2;
    sps2 = (steps + split2 - 1) / split2;
  }
  const int64_t sps_final = sps2;
  pl.split = (int)((steps + sps_final - 1) / sps_final);
  pl.k_slice = sps_final * SK_STEP;
  pl.wk = wk;
  pl.wn = SK_W / wk;
  pl.spw = (int)((sps_final + wk - 1) / wk);
  pl.blocks = blocks;
  pl.x_lds = (int)(sps_final * per_step);
  pl.red_lds = wk > 1 ? (int)red : 0;
  const int64_t lds = pl.x_lds + pl.red_lds;
  const int64_t occ = lds * 2 <= kLds ? 2 : 1;  // workgroups per CU
  int64_t grid = 256 * occ / pl.split / pl.mz;  // workgroups per row block
  if (grid < 1) grid = 1;
  if (grid > pl.blocks) grid = pl.blocks;
  pl.grid = (int)(grid * pl.mz);
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
  const hipError_t e = order == 0 ? launch_skinny_kernels<0>(p, pl, perch, s)
                                  : launch_skinny_kernels<1>(p, pl, perch, s);
  if (e != hipSuccess || pl.split == 1) return e;
  return launch_splitk_reduce(p.partial, p.bias, p.out, p.ldo, p.M, p.N, pl.split, s);
}

}  // namespace q4
