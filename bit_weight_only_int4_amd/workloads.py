"""Seeded synthetic workloads for the weight-only 4-bit linear layer.

This module only draws random inputs; it holds none of the layer's
arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle's checks
take their inputs from here.

Recipe (every tensor is drawn on the CPU from a fresh ``torch.Generator``
seeded with ``seed``, in the order x -> packed bytes -> scales -> bias):
  * x       float32 [M, K]: uniform[a, b] as ``a + (b - a) * rand`` or N(0, 1)
            as ``randn``, per workload.
  * qw      uint8 [N, ceil(K / 2)]: every byte uniform in 0..255, so each
            nibble (including the unused pad nibble of an odd K) is uniform in
            0..15.
  * scales  float32 [ceil(K / gs), N] (grouped) or [N] (per-channel),
            uniform[lo, hi].
  * bias    float32 [N], uniform[-0.1, 0.1], for the workloads that have one.

The shapes are those of the Llama-3.2-1B and Llama-3.1-8B projections that
the pages measure (page 4, "Kernel level"; page 1, the steel and pwdq
entries), drawn synthetically: no model weights are used.

Pages cited by number (the texts this layer is written from):
  page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
          (its stack entries #20730 ... #20801);
  page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
  page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
          (its stack entries #20917 ... #21005);
  page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
  page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
"""
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Projection:
    name: str
    M: int
    K: int
    N: int
    group_size: int            # 0 = per-channel scales [N]
    x_dist: Tuple              # ("uniform", lo, hi) or ("normal",)
    scale_range: Tuple[float, float]
    has_bias: bool = False
    order: str = "low_first"   # nibble order of the packed bytes

    @property
    def Kp(self) -> int:
        return (self.K + 1) // 2

    @property
    def G(self) -> int:
        return 1 if self.group_size == 0 else -(-self.K // self.group_size)

    def with_m(self, M: int) -> "Projection":
        return replace(self, M=M, name=f"{self.name.split('@')[0]}@M{M}")

    # Algorithmic HBM bytes of one call: packed weights, scales, x, out, bias.
    def alg_bytes(self, scale_bytes: int = 4) -> int:
        """scale_bytes: 4 for fp32 scales, 2 for binary16 (q4f16_1)."""
        scale_elems = self.N if self.group_size == 0 else self.G * self.N
        b = self.N * self.Kp + scale_bytes * scale_elems + 4 * self.M * self.K \
            + 4 * self.M * self.N
        if self.has_bias:
            b += 4 * self.N
        return b

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


_U11 = ("uniform", -1.0, 1.0)
_NRM = ("normal",)


def _llama1b(M):
    s = (0.005, 0.02)
    return [
        Projection(f"1b_q_2048x2048@M{M}", M, 2048, 2048, 32, _NRM, s),
        Projection(f"1b_gate_2048x8192@M{M}", M, 2048, 8192, 32, _NRM, s),
        Projection(f"1b_up_2048x8192@M{M}", M, 2048, 8192, 32, _NRM, s),
        Projection(f"1b_down_8192x2048@M{M}", M, 8192, 2048, 32, _NRM, s),
    ]


def _llama8b(M):
    s = (0.002, 0.01)
    return [
        Projection(f"8b_q_4096x4096@M{M}", M, 4096, 4096, 128, _NRM, s),
        Projection(f"8b_gateup_4096x14336@M{M}", M, 4096, 14336, 128, _NRM, s),
        Projection(f"8b_down_14336x4096@M{M}", M, 14336, 4096, 128, _NRM, s),
    ]


def _per_channel():
    s = (0.005, 0.02)
    out = [Projection(f"lm_head_2048x128257@M{M}", M, 2048, 128257, 0, _U11, s,
                      order="high_first") for M in (1, 7, 333)]
    out.append(Projection("odd_k_2008x3000@M65", 65, 2008, 3000, 0, _U11, s,
                          order="high_first"))
    return out


# The five workloads.  Each entry is a list of projections.
CONFIGS = {
    "tiny": [Projection("tiny_256x128@M4", 4, 256, 128, 32, _U11,
                        (0.005, 0.02), has_bias=True)],
    "decode_1b": _llama1b(1),
    "prefill_1b": _llama1b(64) + _llama1b(512) + _llama1b(2048),
    "llama8b_gs128": _llama8b(1) + _llama8b(512),
    "per_channel_edges": _per_channel(),
}


def make_inputs(p: Projection, seed: int = 0, *, bias: Optional[bool] = None):
    """Draw (x, qw, scales, bias) for projection ``p`` as CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if p.x_dist[0] == "uniform":
        lo, hi = p.x_dist[1], p.x_dist[2]
        x = lo + (hi - lo) * torch.rand((p.M, p.K), generator=g,
                                        dtype=torch.float32)
    else:
        x = torch.randn((p.M, p.K), generator=g, dtype=torch.float32)
    qw = torch.randint(0, 256, (p.N, p.Kp), generator=g, dtype=torch.uint8)
    lo, hi = p.scale_range
    sshape = (p.N,) if p.group_size == 0 else (p.G, p.N)
    scales = lo + (hi - lo) * torch.rand(sshape, generator=g,
                                         dtype=torch.float32)
    want_bias = p.has_bias if bias is None else bias
    b = None
    if want_bias:
        b = -0.1 + 0.2 * torch.rand((p.N,), generator=g, dtype=torch.float32)
    return x.contiguous(), qw.contiguous(), scales.contiguous(), b


def small_projection(M, K, N, group_size, *, order="low_first", has_bias=False,
                     x_dist=_NRM, scale_range=(0.005, 0.02), name=None):
    """An ad-hoc projection for parity and edge-case tests."""
    return Projection(name or f"adhoc_M{M}_K{K}_N{N}_gs{group_size}", M, K, N,
                      group_size, x_dist, scale_range, has_bias, order)
