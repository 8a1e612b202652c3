// q4_kernels.h -- host-side interface between the C ABI (q4_abi.hip) and the
// kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4linear.h"

namespace q4 {

struct GemvParams {
  const float* x;
  int64_t ldx;
  const uint8_t* qw;
  int64_t ldq;
  const float* scales;
  const _Float16* scales16;  // binary16 scales instead (q4f16_1), else nullptr
  int64_t lds;
  int64_t group_size;  // 0 = per-channel
  int64_t G;           // number of scale rows (1 for per-channel)
  const float* bias;
  float* out;
  int64_t ldo;
  float* partial;      // split-K workspace [split][M][N] (split > 1)
  int64_t M, N, K;
  int64_t k_per_split; // filled by launch_gemv
  int32_t rows_per_block;
  int32_t split;
  int32_t log2_gs;     // power-of-two group sizes: log2(group_size)
  int32_t waves_k;     // waves per workgroup along K (one 2048*CPL span each)
  int32_t waves_r;     // waves per workgroup along N (R rows each)
  int32_t spans;       // streaming kernel: 2048-wide K spans (ceil(K / 2048))
  int32_t blocks;      // streaming kernel: row blocks of (waves x rows per step) rows
};

// Streaming GEMV (one activation row, aligned shapes): the most workgroups
// a launch runs; a workgroup block is (waves per workgroup) x (rows per wave
// step) rows.
constexpr int kStreamMaxGrid = 1024;

struct GemvPlan {
  int cfg;            // chunks of 32 k per lane (1 or 2)
  int mb;             // activation rows per workgroup (low-batch kernel), 1 = one row
  int waves_k;        // waves per workgroup along K, each over 2048 * cfg k
  int waves_r;        // waves per workgroup along N
  int rows_per_wave;  // R
  int split;
  int64_t k_per_split;
  int rows_per_block;
  int64_t blocks_n;
};

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int64_t group_size);

// scale layouts the GEMV kernels tell apart
namespace gemv {
enum ScaleMode : int { kPerChannel = 0, kStaged = 1, kGeneric = 2 };
}

// The kernel a call runs, as launch_gemv chose it.
struct GemvLaunch {
  dim3 grid;
  int R;       // rows per wave (2, 4, 8)
  int mb;      // activation rows per workgroup (1: one-row kernel)
  bool xl;     // activations through LDS
  int order;   // nibble order
  int smode;   // gemv::ScaleMode
  bool qa4;    // dword-aligned weight rows
  bool sa16;   // vector scale loads
  bool stream; // the streaming kernel (grid.x workgroups loop over row blocks)
  int depth;   // streaming kernel: wave steps in its load ring (1 or 2)
  int waves;   // streaming kernel: waves per workgroup (4 or 8)
};

template <typename ST>
hipError_t launch_gemv_kernels(const GemvParams& p, const GemvLaunch& l, hipStream_t s);
// (instantiated for float and _Float16 in q4_gemv_s32.hip / q4_gemv_s16.hip)

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size);
hipError_t launch_gemv(const GemvParams& p, int order, bool qa4, hipStream_t s);

struct GemmParams {
  const float* x;
  int64_t ldx;
  const uint8_t* qw;
  int64_t ldq;
  const float* scales;
  const _Float16* scales16;  // binary16 scales instead (q4f16_1), else nullptr
  int64_t lds;
  int64_t group_size;  // 0 = per-channel
  int64_t G;
  const float* bias;
  float* out;
  int64_t ldo;
  float* partial;      // split-K workspace [split][M][N] (split > 1)
  _Float16* x16;       // binary16 activations [x16_rows][x16_pitch] (workspace)
  int64_t x16_pitch;
  // pipelined kernel with K % 64 != 0: each row's bytes of the last 64-k step
  // (32 per row, bytes past K as 0x88), written by the binary16 pre-pass into
  // the workspace; else nullptr
  uint8_t* qtail;
  int32_t log2_gs;     // group index by shift (power-of-two group size), else -1
  int64_t M, N, K;
  int64_t k_per_split; // multiple of the K step, filled by launch_gemm
  int32_t split;
  int32_t tiles_m, tiles_n;
};

struct GemmPlan {
  int cfg;
  int split;
  int64_t k_per_split;
  int tiles_m, tiles_n;
  int64_t x16_rows, x16_pitch;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t group_size);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size);
// The GEMM a call runs: the skinny kernel where it applies, else the tiled
// one.  *skinny (if not null) tells which.
hipError_t launch_gemm(const GemmParams& p, int order, bool qa4, void* workspace,
                       hipStream_t s, bool* skinny = nullptr);

// Few-row MFMA GEMM (q4_skinny.hip): 1 <= M <= 1024 (by a measured size rule
// above 32 rows), K % 8 == 0, per-channel or power-of-two groups >= 32,
// dword-aligned weight rows.
struct SkinnyPlan {
  bool ok;          // the sizes are the kernel's
  int mz;           // row blocks (of mrows rows) handled by separate workgroups
  int mrows;        // rows per row block (M when mz == 1, else 32)
  int mb;           // 16-row MFMA blocks per row block (1 or 2)
  int ni;           // 16-column MFMA blocks per wave (2 or 4)
  int wn, wk;       // waves per workgroup along N (16 ni columns each) and along K
  int split;        // K slices (grid.y); > 1 only when a slice's activations exceed LDS
  int64_t k_slice;  // k per slice, a multiple of 128
  int spw;          // 128-k steps per wave and column block
  int64_t blocks;   // column blocks of 16 * ni * wn columns
  int grid;         // workgroups per slice, a multiple of mz (persistent over the column blocks)
  int x_lds;        // LDS bytes of the binary16 activations of a slice
  int red_lds;      // LDS bytes of the partial sums (wk > 1)
};
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t group_size);
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size);
bool skinny_fits(const GemmParams& p, const SkinnyPlan& pl, bool qa4);
hipError_t launch_skinny(const GemmParams& p, const SkinnyPlan& pl, int order, void* workspace,
                         hipStream_t s);
template <int ORDER>
hipError_t launch_skinny_kernels(const GemmParams& p, const SkinnyPlan& pl, bool perch,
                                 hipStream_t s);
// (instantiated for each nibble order in q4_skinny_o0.hip / q4_skinny_o1.hip)

// stage exports
hipError_t launch_unpack_codes(const uint8_t* qw, int64_t ldq, int64_t N,
                               int64_t K, int order, int8_t* codes,
                               int64_t ldc, hipStream_t s);
hipError_t launch_dequant(const uint8_t* qw, int64_t ldq, const float* scales,
                          int64_t lds, int64_t group_size, int64_t N,
                          int64_t K, int order, int dtype, void* w,
                          int64_t ldw, hipStream_t s);

// input gradient (fp32) and re-quantization
struct BwdParams {
  const float* dout;
  int64_t lddo;
  const uint8_t* qw;
  int64_t ldq;
  const float* scales;
  int64_t lds;
  int64_t group_size;  // 0 = per-channel
  float* dx;
  int64_t lddx;
  float* partial;      // [blocks_n][M][K] when blocks_n > 1
  int64_t M, N, K;
  int64_t rows_per_wg; // filled by launch_bwd_f32
  int64_t blocks_n;
  int32_t log2_gs;     // power-of-two group size: log2, else -1
};

struct BwdPlan {
  int mb;              // activation rows per workgroup pass (1, 2, 4)
  int64_t blocks_m, blocks_k, blocks_n;
  int64_t rows_per_wg;
};

BwdPlan plan_bwd(int64_t M, int64_t N, int64_t K);
size_t bwd_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_bwd_f32(const BwdParams& p, int order, bool qa4, hipStream_t s);
hipError_t launch_requant(const float* latent, int64_t ldl, const float* scales, int64_t lds,
                          int64_t gs, int64_t N, int64_t K, int order, uint8_t* qw, int64_t ldq,
                          hipStream_t s);

// input gradient on MFMA (binary16 operands, fp32 accumulation)
struct BwdMfmaParams {
  const _Float16* d16;  // binary16 d_out [mp][np] (workspace), zero-padded
  int64_t d16_pitch;
  const uint8_t* qw;
  int64_t ldq;
  const float* scales;
  int64_t lds;
  int64_t group_size;  // 0 = per-channel; else a multiple of 8
  int32_t log2_gs;     // power-of-two group size: log2, else -1
  float* dx;
  int64_t lddx;
  float* partial;      // [split][M][K] when split > 1 (workspace)
  int64_t M, N, K;
  int64_t n_per_split; // multiple of the N step
  int32_t split;
  int32_t tiles_m, tiles_k;
};

struct BwdMfmaPlan {
  int64_t tiles_m, tiles_k;
  int64_t mp, np;      // padded binary16 d_out
  int64_t n_per_split;
  int split;
};

BwdMfmaPlan plan_bwd_mfma(int64_t M, int64_t N, int64_t K);
size_t bwd_mfma_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_bwd_mfma(const BwdParams& p, int order, bool qa4, void* workspace,
                           hipStream_t s);

// out[m, n] = sum over z of partial[z][m][n] (+ bias[n]), z in order
hipError_t launch_splitk_reduce(const float* partial, const float* bias, float* out, int64_t ldo,
                                int64_t M, int64_t N, int split, hipStream_t s);

__global__ void splitk_reduce_kernel(const float* __restrict__ partial,
                                     const float* __restrict__ bias,
                                     float* __restrict__ out, int64_t ldo,
                                     int64_t M, int64_t N, int split);

}  // namespace q4
