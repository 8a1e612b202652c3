"""Pins of the oracle's input-gradient and re-quantization functions (no GPU).

Input gradient, page 3, "Add fp32 matmul ops (mm, bmm, linear)", stack entry
#20943: d_x[m, k] = sum_n d_out[m, n] * dequant(W)[n, k].  Pinned by a dense
fp64 matmul over a weight the test builds itself, by the adjoint identity
<d_x, x> = <d_out, x W^T> against the forward oracle (a transposed operand or
a swapped index breaks it), by exact special cases and by exact rational
arithmetic.

Re-quantization, page 3, stack entries #20945 and #20946: code =
clamp(round(latent / scale), -8, 7) + 8, zero scale -> code 8, packed into the
flat [N, K/2] layout.  Pinned by the round trip through the dequant stage,
by numpy's ties-to-even rounding on exact ties, by clamping and zero scales,
and by the test-side packer written from the pages' packers.

Binary16 scales (page 4's q4f16_1 weights, read as 4-bit codes with
binary16 group scales): every one of the 65536 bit patterns widens to numpy's
binary16 value, and a worked example computed by hand.

Pages cited by number (the texts this layer is written from):
  page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
          (its stack entries #20730 ... #20801);
  page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
  page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
          (its stack entries #20917 ... #21005);
  page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
  page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
"""
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import q4_oracle as orc
from tests.packing import expand_scales, pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _setup(rng, M, K, N, gs, order):
    raw = rng.integers(0, 16, size=(N, K), dtype=np.int64)
    qw = pack(raw, order, pad=int(rng.integers(0, 16)))
    scales = rng.uniform(0.005, 0.02, N if gs == 0 else (-(-K // gs), N)).astype(np.float32)
    dout = rng.standard_normal((M, N)).astype(np.float32)
    W = (raw - 8).astype(np.float64) * expand_scales(scales, N, K, gs)
    return raw, qw, scales, dout, W


# --------------------------------------------------------------------------
# Input gradient
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,gs,order", [(5, 300, 70, 32, "low_first"),
                                            (1, 2008, 33, 0, "high_first"),
                                            (3, 515, 64, 128, "low_first"),
                                            (2, 64, 129, 8, "high_first")])
def test_backward_dense_matmul(M, K, N, gs, order):
    rng = np.random.default_rng(M * 7 + K + N)
    _, qw, scales, dout, W = _setup(rng, M, K, N, gs, order)
    ref = dout.astype(np.float64) @ W
    dx, den = orc.linear_backward(dout, qw, scales, K=K, group_size=gs, order=order)
    assert dx.shape == (M, K)
    assert np.all(np.abs(dx - ref) <= 1e-12 * den + 1e-300)
    assert np.allclose(den, np.abs(dout.astype(np.float64)) @ np.abs(W), rtol=1e-12)


def test_backward_adjoint_of_forward():
    """<d_x, x> equals <d_out, x W^T> computed by the forward oracle."""
    rng = np.random.default_rng(11)
    M, K, N, gs = 4, 200, 45, 32
    _, qw, scales, dout, _ = _setup(rng, M, K, N, gs, "low_first")
    x = rng.standard_normal((M, K)).astype(np.float32)
    dx, den_b = orc.linear_backward(dout, qw, scales, K=K, group_size=gs)
    y, den_f = orc.linear(x, qw, scales, None, K=K, group_size=gs)
    lhs = float(np.sum(dx * x.astype(np.float64)))
    rhs = float(np.sum(y * dout.astype(np.float64)))
    bound = 1e-12 * (float(np.sum(den_b * np.abs(x))) + float(np.sum(den_f * np.abs(dout))))
    assert abs(lhs - rhs) <= bound


def test_backward_special_cases():
    rng = np.random.default_rng(12)
    M, K, N = 3, 97, 11
    # all nibbles 8: the gradient is exactly zero, and so is the normaliser
    qw = pack(np.full((N, K), 8), "low_first", pad=3)
    scales = rng.uniform(0.005, 0.02, (4, N)).astype(np.float32)
    dout = rng.standard_normal((M, N)).astype(np.float32)
    dx, den = orc.linear_backward(dout, qw, scales, K=K, group_size=32)
    assert np.all(dx == 0) and np.all(den == 0)
    # a one-hot d_out row picks one dequantized weight row, exactly
    raw, qw, scales, _, W = _setup(rng, 1, K, N, 32, "high_first")
    for n in (0, 5, N - 1):
        e = np.zeros((1, N), np.float32)
        e[0, n] = 1.0
        dx, _ = orc.linear_backward(e, qw, scales, K=K, group_size=32, order="high_first")
        assert np.array_equal(dx[0], W[n])


def test_backward_fraction_bruteforce():
    rnd = random.Random(13)
    rng = np.random.default_rng(13)
    for trial in range(30):
        M, N, K = rnd.randint(1, 3), rnd.randint(1, 5), rnd.randint(1, 40)
        gs = rnd.choice([0, 1, 3, 8, 32])
        order = rnd.choice(["low_first", "high_first"])
        raw, qw, scales, dout, _ = _setup(rng, M, K, N, gs, order)
        dx, den = orc.linear_backward(dout, qw, scales, K=K, group_size=gs, order=order)
        for m in range(M):
            for k in range(K):
                acc = Fraction(0)
                dd = Fraction(0)
                for n in range(N):
                    s = scales[n] if gs == 0 else scales[k // gs, n]
                    t = Fraction(float(dout[m, n])) * (int(raw[n, k]) - 8) * Fraction(float(s))
                    acc += t
                    dd += abs(t)
                assert abs(Fraction(dx[m, k]) - acc) <= dd * Fraction(1, 10 ** 14)
                assert abs(Fraction(den[m, k]) - dd) <= dd * Fraction(1, 10 ** 14)


def test_backward_sampled_matches_full():
    rng = np.random.default_rng(14)
    M, K, N, gs = 4, 300, 50, 32
    _, qw, scales, dout, _ = _setup(rng, M, K, N, gs, "low_first")
    dx, den = orc.linear_backward(dout, qw, scales, K=K, group_size=gs)
    ms = rng.integers(0, M, 40)
    ks = rng.integers(0, K, 40)
    v, d = orc.linear_backward_sampled(dout, qw, scales, ms, ks, K=K, group_size=gs)
    assert np.array_equal(v, dx[ms, ks]) and np.array_equal(d, den[ms, ks])


# --------------------------------------------------------------------------
# Re-quantization
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,gs,order", [(256, 32, "low_first"), (2008, 0, "high_first"),
                                        (1001, 8, "low_first"), (7, 3, "high_first")])
def test_requant_round_trip(K, gs, order):
    """latent = RN32(c * s) re-quantizes to the codes it came from (the
    pages build their golden latents as code * scale for this reason)."""
    rng = np.random.default_rng(K + gs)
    N = 37
    raw = rng.integers(0, 16, size=(N, K), dtype=np.int64)
    qw = pack(raw, order, pad=8)
    scales = rng.uniform(0.001, 0.05, N if gs == 0 else (-(-K // gs), N)).astype(np.float32)
    latent = orc.dequant_f32(qw, scales, K, gs, order)
    back = orc.requant(latent, scales, group_size=gs, order=order)
    assert np.array_equal(back, qw)


def test_requant_ties_to_even_and_clamp():
    """Quotients k + 1/2 are exact for power-of-two scales: the codes follow
    numpy's round (ties to even); quotients beyond [-8, 7] clamp."""
    s = np.float32(0.125)
    q = np.array([-9.5, -8.5, -8.0, -7.5, -2.5, -1.5, -0.5, -0.25, 0.0, 0.25, 0.5,
                  1.5, 2.5, 3.5, 6.5, 7.0, 7.5, 8.5, 1e6, -1e6], dtype=np.float64)
    latent = (q * 0.125).astype(np.float32)[None, :]
    assert np.array_equal(latent.astype(np.float64) / 0.125, q[None, :])
    qw = orc.requant(latent, np.array([s], np.float32), group_size=0)
    expect = np.clip(np.round(q), -8, 7).astype(np.int64) + 8
    codes = orc.unpack_codes(qw, q.size) + 8
    assert np.array_equal(codes[0], expect)


def test_requant_zero_scale_and_nan():
    latent = np.array([[1.0, -3.0, np.inf, np.nan, 0.0, 5.0]], np.float32)
    qw = orc.requant(latent, np.zeros((1, 1), np.float32), group_size=6)
    assert np.array_equal(orc.unpack_codes(qw, 6), np.zeros((1, 6), np.int8))
    # a NaN quotient under a nonzero scale also gives code 8; +-inf clamps
    s = np.array([0.5], np.float32)
    qw = orc.requant(latent, s, group_size=0)
    assert orc.unpack_codes(qw, 6).tolist() == [[2, -6, 7, 0, 0, 7]]


def test_requant_packing_against_test_packer():
    """Layout and nibble order match the packers of the pages (tests/packing.py),
    including the code-8 pad nibble of an odd K and untouched row padding."""
    rng = np.random.default_rng(15)
    N, K, gs = 9, 67, 16
    scales = rng.uniform(0.01, 0.02, (-(-K // gs), N)).astype(np.float32)
    latent = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    S = expand_scales(scales, N, K, gs, np.float32)
    codes = np.clip(np.round((latent / S).astype(np.float64)), -8, 7).astype(np.int64) + 8
    for order in ("low_first", "high_first"):
        got = orc.requant(latent, scales, group_size=gs, order=order, ldq=40, fill=0xAB)
        want = pack(codes, order, pad=8, ldq=40)
        assert np.array_equal(got[:, :34], want[:, :34])
        assert np.all(got[:, 34:] == 0xAB)


def test_requant_golden():
    with open(GOLDEN) as f:
        g = json.load(f)["requant"]
    latent = np.array(g["latent"], np.float32)
    scales = np.array(g["scales"], np.float32)
    for order, want in g["bytes"].items():
        got = orc.requant(latent, scales, group_size=g["group_size"], order=order)
        assert got.tolist() == want, order


# --------------------------------------------------------------------------
# Binary16 scales
# --------------------------------------------------------------------------

def test_f16_scale_values_every_pattern():
    """All 65536 binary16 patterns widen to the value numpy's binary16 type
    gives them (normal, subnormal, signed zero, infinities; NaN stays NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_scales_to_f32(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_f16_scales_worked_example():
    """K = 4, group size 2, one row.  Codes 9, 7, 15, 0 (c = 1, -1, 7, -8),
    x = (1, 2, 3, 4), scales 0.5 (0x3800) and 2.0 (0x4000):
    0.5 * (1 - 2) + 2 * (21 - 32) = -22.5.  A second row with scales -2^-24
    (0x8001, the smallest subnormal) and 65504 (0x7BFF) and all codes 15
    (c = 7): -2^-24 * 7 * 3 + 65504 * 7 * 7 = 3209696 - 21 * 2^-24."""
    x = np.array([[1, 2, 3, 4]], np.float32)
    raw = np.array([[9, 7, 15, 0], [15, 15, 15, 15]])
    bits = np.array([[0x3800, 0x8001], [0x4000, 0x7BFF]], np.uint16)
    want = np.array([[-22.5, 3209696.0 - 21.0 * 2.0 ** -24]])
    for order in ("low_first", "high_first"):
        out, den = orc.linear_f16_scales(x, pack(raw, order), bits, K=4, group_size=2,
                                         order=order)
        assert np.array_equal(out, want), order
        assert den[0, 0] == 0.5 * (1 + 2) + 2 * (21 + 32)
