// q4_device.h -- device-side building blocks shared by every gfx950 kernel of
// the weight-only 4-bit linear layer: nibble unpack, the signed offset, and
// the binary16 dequant.  The layer's kernels and the stage-export kernels
// (q4_unpack_codes / q4_dequant) call these same functions, so the exported
// stages are the arithmetic the layer runs.
//
// Packed layout: row n of the weight holds ceil(K/2) bytes; a 32-bit word at
// byte offset 4*d of the row holds k = 8d .. 8d+7.  Nibble i of the word
// (bits 4i .. 4i+3) is k = 8d + i for the q4gsw packer ((odd << 4) | even,
// even k low) and k = 8d + (i ^ 1) for the qcs4w packer ((even << 4) | odd);
// page 5, "[ExecuTorch][WebGPU] Add linear_qcs4w op", Constraints (2).
// The signed value is c = q - 8 in [-8, 7]: page 3, "Add fp32 matmul ops
// (mm, bmm, linear)", stack entry #20943.
//
// Pages cited by number (the texts this layer is written from):
//   page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
//           (its stack entries #20730 ... #20801);
//   page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
//   page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
//           (its stack entries #20917 ... #21005);
//   page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
//   page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte vector that is only guaranteed 4-byte aligned: gfx950 serves it
// with one global_load_dwordx4 (dword alignment suffices for global memory).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));  // 8-byte aligned

enum Order : int { kLowFirst = 0, kHighFirst = 1 };

// A loop-invariant constant held in a VGPR.  VOP3 encodings on gfx9 take no
// literal and at most one SGPR, so keeping the OR-mask in a VGPR lets the
// compiler fuse (w & mask) | magic into a single v_and_or_b32.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

struct Magic {
  uint32_t lo;  // 0x6400 per half: binary16 1024.0, nibble in fraction bits 0..3
  uint32_t hi;  // 0x5400 per half: binary16 64.0, nibble in fraction bits 4..7
  __device__ __forceinline__ static Magic make() {
    return Magic{vgpr_const(0x64006400u), vgpr_const(0x54005400u)};
  }
};

// Unpack one packed word into its eight signed values as four binary16 pairs.
// Pair p holds nibbles (p, p + 4) of the word: half .x = nibble p, .y =
// nibble p + 4.  Exact: 1024 + q and 64 + q are exact binary16 integers, and
// subtracting 1032 / 72 leaves q - 8 exactly.
__device__ __forceinline__ void unpack_word(uint32_t w, const Magic& mg,
                                            h2 (&c)[4]) {
  const uint32_t w8 = w >> 8;
  const uint32_t t0 = (w & 0x000F000Fu) | mg.lo;   // nibbles 0, 4
  const uint32_t t1 = (w & 0x00F000F0u) | mg.hi;   // nibbles 1, 5
  const uint32_t t2 = (w8 & 0x000F000Fu) | mg.lo;  // nibbles 2, 6
  const uint32_t t3 = (w8 & 0x00F000F0u) | mg.hi;  // nibbles 3, 7
  const h2 b_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 b_hi = {(_Float16)72.0f, (_Float16)72.0f};
  c[0] = __builtin_bit_cast(h2, t0) - b_lo;
  c[1] = __builtin_bit_cast(h2, t1) - b_hi;
  c[2] = __builtin_bit_cast(h2, t2) - b_lo;
  c[3] = __builtin_bit_cast(h2, t3) - b_hi;
}

// Offset (0..7) within the word's eight k of nibble i.
template <int ORDER>
__device__ __forceinline__ constexpr int nibble_k(int i) {
  return ORDER == kLowFirst ? i : (i ^ 1);
}

// Offset within the word's eight k of half h (0 = .x, 1 = .y) of pair p.
template <int ORDER>
__device__ __forceinline__ constexpr int pair_k(int p, int h) {
  return nibble_k<ORDER>(p + 4 * h);
}

// Binary16 dequant of a pair: RN16(c * s16), with s16 = RN16(s) given as a
// pair.  c * s16 needs at most 15 significant bits, so the single IEEE
// multiply rounds the exact product once.
__device__ __forceinline__ h2 dequant_pair_f16(h2 c, h2 s16) { return c * s16; }

__device__ __forceinline__ h2 splat_f16(float s) {
  const _Float16 h = (_Float16)s;  // v_cvt_f16_f32: round to nearest even
  return h2{h, h};
}

// Element i of a scale array held either as fp32 (s16 == nullptr) or as
// binary16 (q4f16_1 weights), widened exactly.  The choice comes from a
// kernel argument, so the branch is wave-uniform.
__device__ __forceinline__ float scale_at(const float* s32, const _Float16* s16, int64_t i) {
  return s16 ? (float)s16[i] : s32[i];
}

// Raw code (0..15) of nibble k of a row, one byte at a time (used by the
// stage-export kernels and for ragged tails).
template <int ORDER>
__device__ __forceinline__ int raw_code_at(const uint8_t* row, int64_t k) {
  const uint32_t b = row[k >> 1];
  const int odd = (int)(k & 1);
  const int shift = (ORDER == kLowFirst) ? (odd ? 4 : 0) : (odd ? 0 : 4);
  return (int)((b >> shift) & 0xFu);
}

// XCD-aware block order.  The hardware hands consecutive workgroup ids to
// the 8 XCDs round-robin; this maps them back so that each XCD gets one
// contiguous range of logical tiles, which then share that XCD's L2 (the
// neighbouring rows of the scale matrix sit in the same cache lines).
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = nblocks / kXcd;
  const uint32_t rem = nblocks % kXcd;
  const uint32_t xcd = bid % kXcd;
  const uint32_t idx = bid / kXcd;
  // XCDs 0 .. rem-1 own per + 1 logical blocks, the rest own per.
  const uint32_t start = xcd * per + (xcd < rem ? xcd : rem);
  return start + idx;
}

}  // namespace q4
