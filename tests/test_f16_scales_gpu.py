"""GPU parity of the binary16-scale layer (q4_linear_f16_scales) against the
fp64 oracle, through the C ABI.

Page 4 runs its decode GEMVs on q4f16_1 weights, read here as 4-bit codes
with binary16 group scales.  The oracle widens each binary16 scale exactly
and evaluates the layer; the bar is the layer's own (1e-5 on the fp32 GEMV
paths, 2e-3 on the binary16 MFMA GEMM, normalised by sum_k |x * w|).  Cases
cover every kernel the entry can run: the decode GEMV (staged, per-channel
and any-group-size scales), the low-batch GEMV, the pipelined GEMM (its
binary16 scale fetch needs even N and an even scale pitch) and the general
GEMM (odd N, odd pitch, ragged K).
"""
import zlib

import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs, small_projection
from oracle import q4_oracle as orc
from tests.gpu_util import TOL, log, need_gpu, normalised_error, run_gpu
from tests.packing import pack

pytestmark = pytest.mark.gpu


def _bits(s16: torch.Tensor) -> np.ndarray:
    return s16.contiguous().view(torch.int16).numpy().view(np.uint16)


def _case(M, K, N, gs, *, order="low_first", math="auto", pad=(0, 0, 0, 0), bias=False,
          seed=0, expect=None):
    log(f"[f16 scales] M={M} K={K} N={N} gs={gs} order={order} math={math} pad={pad}")
    p = small_projection(M, K, N, gs, order=order, has_bias=bias, x_dist=("uniform", -1, 1))
    x, qw, s, bb = make_inputs(p, seed)
    s16 = s.half()
    out, path, guards = run_gpu(x, qw, s16, bb, K=K, gs=gs, order=order, math=math, pad=pad)
    ref, den = orc.linear_f16_scales(x.numpy(), qw.numpy(), _bits(s16),
                                     None if bb is None else bb.numpy(), K=K, group_size=gs,
                                     order=order)
    assert guards, "write outside [M, N]"
    assert not np.any(np.isnan(out))
    err = normalised_error(out, ref, den)
    log(f"           path={path} max normalised error={err:.3e} (tol {TOL[path]:.0e})")
    assert err <= TOL[path]
    if expect:
        assert path == expect
    return out


@pytest.mark.parametrize("M,K,N,gs,order,math,pad,expect", [
    # decode GEMV: staged groups (vector scale loads), per-channel, other sizes
    (1, 2048, 515, 32, "low_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    (1, 8192, 1000, 128, "high_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    (1, 2008, 301, 0, "high_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    (1, 1000, 130, 24, "low_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    (1, 2007, 257, 32, "low_first", "auto", (1, 3, 1, 2), "gemv_f32"),
    (1, 65536, 64, 32, "low_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    # low batch
    (4, 2048, 300, 32, "low_first", "auto", (0, 0, 0, 0), "gemv_f32"),
    (7, 2048, 1000, 0, "high_first", "f32", (0, 0, 0, 0), "gemv_f32"),
    (3, 4096, 257, 64, "high_first", "f32", (0, 0, 2, 0), "gemv_f32"),
    # low batch over four spans of K: K split in two, four rows per workgroup
    (4, 8192, 515, 32, "low_first", "f32", (0, 0, 0, 0), "gemv_f32"),
    (12, 8192, 300, 128, "high_first", "f32", (0, 0, 2, 0), "gemv_f32"),
    # few-row MFMA GEMM: per-channel, grouped with a scale pitch, K split
    (7, 2048, 1000, 0, "high_first", "auto", (0, 0, 0, 0), "gemm_f16_skinny"),
    (24, 4096, 600, 128, "low_first", "auto", (0, 0, 2, 0), "gemm_f16_skinny"),
    (16, 8192, 301, 32, "high_first", "f16", (0, 0, 1, 0), "gemm_f16_skinny"),
    # pipelined GEMM (aligned, even N and pitch), several tiles and ragged M
    (70, 1024, 4136, 32, "low_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (1100, 2048, 512, 64, "high_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (1100, 2048, 700, 0, "low_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (129, 8192, 2048, 32, "low_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    # general GEMM: odd N, odd scale pitch, ragged K, small groups
    (1100, 2048, 257, 32, "low_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (1100, 2048, 300, 32, "high_first", "f16", (0, 0, 1, 0), "gemm_f16"),
    # few-row GEMM over three row blocks, and K % 32 != 0 with factored scales
    (65, 2048, 300, 32, "high_first", "f16", (0, 0, 1, 0), "gemm_f16_skinny"),
    (65, 2008, 3000, 0, "high_first", "auto", (0, 0, 0, 0), "gemm_f16_skinny"),
    (7, 2008, 300, 128, "low_first", "f16", (0, 0, 2, 0), "gemm_f16_skinny"),
    (40, 2007, 300, 32, "low_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (17, 300, 77, 8, "high_first", "f16", (0, 0, 0, 0), "gemm_f16"),
    (513, 1024, 260, 100, "low_first", "auto", (0, 0, 0, 0), "gemm_f16"),
])
def test_f16_scales_parity(M, K, N, gs, order, math, pad, expect):
    need_gpu()
    _case(M, K, N, gs, order=order, math=math, pad=pad, bias=(M % 2 == 1),
          seed=M * 131 + N, expect=expect)


@pytest.mark.parametrize("math,M", [("f32", 1), ("f32", 5), ("f16", 1), ("f16", 70),
                                    ("auto", 200)])
def test_f16_scales_integer_case_is_exact(math, M):
    """x in {-2..2} and binary16 scales 2^-6: every path equals the oracle
    bit for bit (as for fp32 scales)."""
    need_gpu()
    rng = np.random.default_rng(M + 7)
    K, N = 2048, 302
    raw = rng.integers(0, 16, size=(N, K))
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    qw = torch.from_numpy(pack(raw, "low_first"))
    s16 = torch.full((K // 32, N), 2.0 ** -6, dtype=torch.float16)
    out, path, guards = run_gpu(x, qw, s16, None, K=K, gs=32, order="low_first", math=math)
    ref, _ = orc.linear_f16_scales(x.numpy(), qw.numpy(), _bits(s16), K=K, group_size=32)
    assert guards
    assert np.array_equal(out.astype(np.float64), ref), path


def test_f16_scales_match_widened_fp32_scales():
    """The binary16 entry gives bit-identical outputs to q4_linear run on the
    same scales widened to fp32, on every kernel (same operands, same
    order)."""
    need_gpu()
    for M, K, N, gs, math in ((1, 2048, 515, 32, "auto"), (4, 2048, 300, 32, "auto"),
                              (130, 2048, 512, 64, "f16"), (96, 2048, 257, 32, "f16")):
        p = small_projection(M, K, N, gs)
        x, qw, s, _ = make_inputs(p, 3)
        s16 = s.half()
        a, pa, _ = run_gpu(x, qw, s16, None, K=K, gs=gs, order="low_first", math=math)
        c, pc, _ = run_gpu(x, qw, s16.float(), None, K=K, gs=gs, order="low_first", math=math)
        assert pa == pc
        assert np.array_equal(a, c), (M, K, N, gs, math)


@pytest.mark.parametrize("name", ["decode_1b", "llama8b_gs128", "per_channel_edges"])
def test_f16_scales_full_size_sampled(name):
    """Each projection of a workload at full size (its M), with its scales
    rounded to binary16, on 300 outputs sampled and computed one by one by
    the oracle."""
    need_gpu()
    dev = torch.device("cuda")
    for p in CONFIGS[name]:
        seed = zlib.crc32(p.name.encode())
        log(f"[f16 scales full] {p.name} seed={seed}")
        x, qw, s, bb = make_inputs(p, seed)
        s16 = s.half()
        out, path = b.linear(x.to(dev), qw.to(dev), s16.to(dev),
                             None if bb is None else bb.to(dev), K=p.K,
                             group_size=p.group_size, nibble_order=p.order, return_path=True)
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed)
        ms = rng.integers(0, p.M, 300)
        ns = rng.integers(0, p.N, 300)
        ref, den = orc.linear_sampled(x.numpy(), qw.numpy(), orc.f16_scales_to_f32(_bits(s16)),
                                      None if bb is None else bb.numpy(), ms, ns, K=p.K,
                                      group_size=p.group_size, order=p.order)
        err = normalised_error(out.cpu().numpy()[ms, ns], ref, den)
        log(f"           path={path} max normalised error={err:.3e}")
        assert err <= TOL[path]
