"""Test-side packer: builds packed weight bytes from chosen codes.

Written from the packers the pages describe (page 5, "Add linear_qcs4w op",
Constraints (2)), not from any unpacker:
  * q4gsw packer ("low_first"):  byte = (code[odd k] << 4) | code[even k]
  * qcs4w packer ("high_first"): byte = (code[even k] << 4) | code[odd k]
For an odd K the last byte's unused nibble is ``pad`` (0..15).

Pages cited by number (the texts this layer is written from):
  page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
          (its stack entries #20730 ... #20801);
  page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
  page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
          (its stack entries #20917 ... #21005);
  page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
  page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
"""
import numpy as np


def pack(codes: np.ndarray, order: str = "low_first", pad: int = 0,
         ldq: int = None) -> np.ndarray:
    """codes: uint8/int array [N, K] of raw codes 0..15 -> uint8 [N, ldq]."""
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    if codes.size and (codes.min() < 0 or codes.max() > 15):
        raise ValueError("raw codes must lie in 0..15")
    Kp = (K + 1) // 2
    ldq = Kp if ldq is None else ldq
    even = codes[:, 0::2]
    odd = np.full((N, Kp), pad, dtype=np.int64)
    odd[:, : K // 2] = codes[:, 1::2]
    if order == "low_first":
        b = (odd << 4) | even
    elif order == "high_first":
        b = (even << 4) | odd
    else:
        raise ValueError(order)
    out = np.zeros((N, ldq), dtype=np.uint8)
    out[:, :Kp] = b.astype(np.uint8)
    return out


def expand_scales(scales: np.ndarray, N: int, K: int, group_size: int,
                  dtype=np.float64) -> np.ndarray:
    """Per-weight scale matrix [N, K]: page 5's index (k // gs) * lds + n,
    or scales[n] when group_size == 0."""
    scales = np.asarray(scales)
    if group_size == 0:
        return np.repeat(scales[:N, None].astype(dtype), K, axis=1)
    g = np.arange(K) // group_size
    return scales[g][:, :N].T.astype(dtype)
