"""Pins of the fp64 CPU oracle against facts fixed by the pages and by
mathematics (no GPU needed).

Each test names what it pins; together they are chosen so that a plausible
mistake in the oracle (swapped nibbles, a wrong signed offset, a transposed
scale index, a dropped bias, a K-tail that reads the pad nibble) fails at
least one of them.

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
import torch

from oracle import q4_oracle as orc
from tests.packing import expand_scales, pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rand_codes(rng, N, K):
    return rng.integers(0, 16, size=(N, K), dtype=np.int64)


# --------------------------------------------------------------------------
# Hand-worked examples (tests/golden/worked_examples.json, cited there).
# --------------------------------------------------------------------------
def test_golden_worked_examples():
    with open(GOLDEN) as f:
        g = json.load(f)
    qw = np.array(g["qw"], dtype=np.uint8)
    x = np.array(g["x"], dtype=np.float32)
    for case in g["cases"]:
        K, gs, order = case["K"], case["group_size"], case["order"]
        scales = np.array(case["scales"], dtype=np.float32)
        bias = None if case["bias"] is None else np.array(case["bias"], np.float32)
        codes = orc.unpack_codes(qw, K, order)
        assert codes.tolist() == case["codes"], case["name"]
        out, den = orc.linear(x, qw, scales, bias, K=K, group_size=gs, order=order)
        assert out.tolist() == case["out"], case["name"]
        assert den.tolist() == case["den"], case["name"]


# --------------------------------------------------------------------------
# P1: unpack order, every byte value, both orders (page 5 packers).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_p1_every_byte_both_orders(order):
    pairs = np.array([(e, o) for e in range(16) for o in range(16)])
    qw = pack(pairs, order)                      # N = 256 rows, K = 2
    assert sorted(qw[:, 0].tolist()) == list(range(256))
    x = np.eye(2, dtype=np.float32)
    scales = np.ones(256, dtype=np.float32)
    out, _ = orc.linear(x, qw, scales, None, K=2, group_size=0, order=order)
    assert np.array_equal(out[0], pairs[:, 0] - 8.0)
    assert np.array_equal(out[1], pairs[:, 1] - 8.0)
    codes = orc.unpack_codes(qw, 2, order)
    assert np.array_equal(codes, pairs - 8)


# --------------------------------------------------------------------------
# P2: all nibbles 8 (byte 0x88, the zero-weight byte of page 3, #20945): the
# output is exactly the bias, and the normaliser is exactly zero.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,gs", [(64, 32), (33, 8), (40, 0), (7, 3)])
def test_p2_all_eights_give_bias(K, gs):
    rng = np.random.default_rng(1)
    M, N = 5, 9
    qw = np.full((N, (K + 1) // 2), 0x88, dtype=np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    scales = (rng.random((N,)) if gs == 0 else
              rng.random((-(-K // gs), N))).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    for order in ("low_first", "high_first"):
        out, den = orc.linear(x, qw, scales, bias, K=K, group_size=gs, order=order)
        assert np.array_equal(out, np.broadcast_to(bias.astype(np.float64), (M, N)))
        assert np.all(den == 0)
        out0, _ = orc.linear(x, qw, scales, None, K=K, group_size=gs, order=order)
        assert np.all(out0 == 0)


# --------------------------------------------------------------------------
# P3: scale indexing with one-hot activations and distinct powers of two.
# Every output is one exact product c * s, so every index is recovered.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,N,gs,lds", [(12, 5, 4, 7), (10, 3, 4, 3),
                                        (9, 4, 0, 0), (16, 6, 16, 6),
                                        (11, 2, 1, 5)])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_p3_scale_indexing(K, N, gs, lds, order):
    rng = np.random.default_rng(K * 100 + N)
    raw = _rand_codes(rng, N, K)
    qw = pack(raw, order, pad=int(rng.integers(0, 16)))
    if gs == 0:
        scales = np.array([2.0 ** (n - 3) for n in range(N)], dtype=np.float32)
    else:
        G = -(-K // gs)
        scales = np.array([[2.0 ** (g * lds + n - 20) for n in range(lds)]
                           for g in range(G)], dtype=np.float32)
    x = np.eye(K, dtype=np.float32)              # row m is e_m
    out, _ = orc.linear(x, qw, scales, None, K=K, group_size=gs, order=order)
    for k in range(K):
        for n in range(N):
            s = scales[n] if gs == 0 else scales[k // gs, n]
            assert out[k, n] == float(raw[n, k] - 8) * float(s), (k, n)


# --------------------------------------------------------------------------
# P4: integer special case.  x in {-2..2}, scales 2^-6: every product and
# partial sum is an exact multiple of 2^-6, so the result is the integer
# matrix product (numpy int64 matmul over the test's own codes) times 2^-6.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,gs", [(3, 64, 17, 32), (5, 2008, 9, 0),
                                      (2, 1001, 6, 128), (4, 96, 40, 8)])
def test_p4_exact_integer_case(M, K, N, gs):
    rng = np.random.default_rng(M * K + N)
    raw = _rand_codes(rng, N, K)
    xi = rng.integers(-2, 3, size=(M, K))
    bias_i = rng.integers(-50, 51, size=N)
    qw = pack(raw, "low_first", pad=15)
    scales = np.full(N if gs == 0 else (-(-K // gs), N), 2.0 ** -6, np.float32)
    out, _ = orc.linear(xi.astype(np.float32), qw, scales,
                        (bias_i * 2.0 ** -6).astype(np.float32),
                        K=K, group_size=gs, order="low_first")
    exact = (xi @ (raw - 8).T + bias_i[None, :]) * 2.0 ** -6
    assert np.array_equal(out, exact)


# --------------------------------------------------------------------------
# P5: linearity in the scale.  Scaling every scale by 2^j scales (out - bias)
# by exactly 2^j; a general factor holds to rounding.
# --------------------------------------------------------------------------
def test_p5_linear_in_scale():
    rng = np.random.default_rng(5)
    M, K, N, gs = 4, 256, 33, 32
    raw = _rand_codes(rng, N, K)
    qw = pack(raw)
    x = rng.standard_normal((M, K)).astype(np.float32)
    scales = rng.uniform(0.005, 0.02, (K // gs, N)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    # without bias the power-of-two relation is exact; the bias is added in
    # fp64 after the sum, so with bias it holds to one rounding of the sum.
    base, den = orc.linear(x, qw, scales, None, K=K, group_size=gs)
    for j in (-3, 1, 5):
        s2 = scales * np.float32(2.0 ** j)
        out, _ = orc.linear(x, qw, s2, None, K=K, group_size=gs)
        assert np.array_equal(out, base * 2.0 ** j)
        outb, _ = orc.linear(x, qw, s2, bias, K=K, group_size=gs)
        assert np.all(np.abs(outb - (base * 2.0 ** j + bias)) <= 1e-15 * (np.abs(outb) + 1))
    f = 1.37
    sf = (scales.astype(np.float64) * f).astype(np.float32)
    out, _ = orc.linear(x, qw, sf, None, K=K, group_size=gs)
    nob, _ = orc.linear(x, qw, scales, None, K=K, group_size=gs)
    # scales are rounded to fp32 after the factor: 2^-24 relative per scale
    assert np.all(np.abs(out - f * nob) <= 1e-6 * den * f + 1e-300)


# --------------------------------------------------------------------------
# P6: identity-like weight.  N = K, code 9 on the diagonal and 8 elsewhere:
# out[m, n] = x[m, n] * s[g(n), n] (+ bias[n]), exactly.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,gs,order", [(64, 16, "low_first"),
                                        (37, 0, "high_first"),
                                        (50, 8, "high_first")])
def test_p6_identity_like(K, gs, order):
    rng = np.random.default_rng(K)
    raw = np.full((K, K), 8, dtype=np.int64)
    np.fill_diagonal(raw, 9)
    qw = pack(raw, order, pad=3)
    M = 3
    x = rng.standard_normal((M, K)).astype(np.float32)
    scales = rng.uniform(0.5, 2.0, K if gs == 0 else (-(-K // gs), K)).astype(np.float32)
    bias = rng.standard_normal(K).astype(np.float32)
    out, _ = orc.linear(x, qw, scales, bias, K=K, group_size=gs, order=order)
    s_diag = scales if gs == 0 else scales[np.arange(K) // gs, np.arange(K)]
    expect = x.astype(np.float64) * s_diag.astype(np.float64)[None, :] + bias
    assert np.array_equal(out, expect)


# --------------------------------------------------------------------------
# P7: textbook reduction.  The dense fp64 linear form of page 2 (a numpy
# matmul over the weight matrix the test builds from its own codes and
# scales) agrees to fp64 rounding.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,gs,order", [(7, 300, 50, 32, "low_first"),
                                            (3, 2008, 31, 0, "high_first"),
                                            (1, 515, 64, 128, "low_first"),
                                            (9, 64, 65, 8, "high_first")])
def test_p7_dense_matmul(M, K, N, gs, order):
    rng = np.random.default_rng(M + K + N)
    raw = _rand_codes(rng, N, K)
    qw = pack(raw, order, pad=int(rng.integers(0, 16)))
    x = rng.standard_normal((M, K)).astype(np.float32)
    scales = rng.uniform(0.005, 0.02, N if gs == 0 else (-(-K // gs), N)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    W = (raw - 8).astype(np.float64) * expand_scales(scales, N, K, gs)
    ref = x.astype(np.float64) @ W.T + bias.astype(np.float64)
    out, den = orc.linear(x, qw, scales, bias, K=K, group_size=gs, order=order)
    assert np.all(np.abs(out - ref) <= 1e-12 * den)
    assert np.allclose(den, np.abs(x.astype(np.float64)) @ np.abs(W).T, rtol=1e-12)
    w64 = orc.dequant_f64(qw, scales, K, gs, order)
    assert np.array_equal(w64, W)


# --------------------------------------------------------------------------
# P8: metamorphic relations.
# --------------------------------------------------------------------------
def test_p8_metamorphic():
    rng = np.random.default_rng(8)
    M, K, N = 6, 96, 20
    raw = _rand_codes(rng, N, K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    # (a) swapping the two nibbles of every byte flips the order
    qlow = pack(raw, "low_first")
    swapped = ((qlow >> 4) | (qlow << 4)).astype(np.uint8)
    s_pc = rng.uniform(0.005, 0.02, N).astype(np.float32)
    a, _ = orc.linear(x, qlow, s_pc, bias, K=K, group_size=0, order="low_first")
    b, _ = orc.linear(x, swapped, s_pc, bias, K=K, group_size=0, order="high_first")
    assert np.array_equal(a, b)
    # (b) per-channel equals grouped with one group (gs == K, or gs > K)
    for gs in (K, K + 5, 10 * K):
        c, _ = orc.linear(x, qlow, s_pc[None, :].copy(), bias, K=K,
                          group_size=gs, order="low_first")
        assert np.array_equal(a, c)
    # (c) permuting weight rows, scales and bias permutes output columns
    perm = rng.permutation(N)
    s_g = rng.uniform(0.005, 0.02, (K // 32, N)).astype(np.float32)
    d, _ = orc.linear(x, qlow, s_g, bias, K=K, group_size=32)
    e, _ = orc.linear(x, np.ascontiguousarray(qlow[perm]),
                      np.ascontiguousarray(s_g[:, perm]),
                      np.ascontiguousarray(bias[perm]), K=K, group_size=32)
    assert np.array_equal(d[:, perm], e)


# --------------------------------------------------------------------------
# P9: brute force in exact rational arithmetic on tiny inputs.
# --------------------------------------------------------------------------
def test_p9_fraction_bruteforce():
    rnd = random.Random(9)
    rng = np.random.default_rng(9)
    for trial in range(40):
        M, N = rnd.randint(1, 4), rnd.randint(1, 4)
        K = rnd.randint(1, 64)
        gs = rnd.choice([0, 1, 2, 3, 8, 32, 64, 100])
        order = rnd.choice(["low_first", "high_first"])
        raw = _rand_codes(rng, N, K)
        qw = pack(raw, order, pad=int(rng.integers(0, 16)))
        x = rng.standard_normal((M, K)).astype(np.float32)
        scales = rng.uniform(0.001, 0.05, N if gs == 0 else (-(-K // gs), N)).astype(np.float32)
        bias = rng.uniform(-1, 1, N).astype(np.float32) if trial % 2 else None
        out, den = orc.linear(x, qw, scales, bias, K=K, group_size=gs, order=order)
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                dd = Fraction(0)
                for k in range(K):
                    s = scales[n] if gs == 0 else scales[k // gs, n]
                    t = Fraction(float(x[m, k])) * (int(raw[n, k]) - 8) * Fraction(float(s))
                    acc += t
                    dd += abs(t)
                if bias is not None:
                    acc += Fraction(float(bias[n]))
                assert abs(Fraction(out[m, n]) - acc) <= Fraction(1, 10 ** 14) * dd \
                    + (abs(acc) * Fraction(1, 2 ** 52))
                assert abs(Fraction(den[m, n]) - dd) <= dd * Fraction(1, 10 ** 14)


# --------------------------------------------------------------------------
# Bit-exact stage references against the library's IEEE conversions.
# --------------------------------------------------------------------------
def test_rn_f16_matches_torch_conversion():
    rng = np.random.default_rng(16)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, -65520.0, 7e4,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 6.1e-5,
            5.9e-8, 1e-9, float("inf"), -float("inf")]
    # exact ties between neighbouring binary16 values at many exponents
    for e in range(-24, 16):
        for f in (1, 3, 5, 1023, 2047):
            vals.append((1024 + f / 2.0) * 2.0 ** (e - 10) if e >= -14
                        else (f / 2.0) * 2.0 ** -24)
    rand = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        rng.uniform(-70000, 70000, 5000)]).astype(np.float32)
    v = np.concatenate([np.array(vals, dtype=np.float32), rand])
    ours = orc.rn_f16_bits(v)
    ref = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = orc.rn_f16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0
    for h in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC800, 0x8001):
        assert orc.f16_value(h) == float(np.array([h], np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("gs,order", [(32, "low_first"), (0, "high_first"), (8, "low_first")])
def test_dequant_stages_match_library_products(gs, order):
    rng = np.random.default_rng(gs + 3)
    N, K = 40, 200
    raw = _rand_codes(rng, N, K)
    qw = pack(raw, order)
    # wide scale range, including values whose products overflow binary16
    shape = N if gs == 0 else (-(-K // gs), N)
    scales = (rng.uniform(0.5, 2.0, shape) * 10.0 ** rng.integers(-8, 5, shape)).astype(np.float32)
    S = torch.from_numpy(expand_scales(scales, N, K, gs, dtype=np.float32))
    C = torch.from_numpy(raw - 8)
    assert np.array_equal(orc.unpack_codes(qw, K, order), (raw - 8).astype(np.int8))
    w32 = orc.dequant_f32(qw, scales, K, gs, order)
    assert np.array_equal(w32.view(np.uint32), (C.float() * S).numpy().view(np.uint32))
    w16 = orc.dequant_f16_bits(qw, scales, K, gs, order)
    ref16 = (C.to(torch.float16) * S.to(torch.float16)).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w16, ref16)


# --------------------------------------------------------------------------
# Layout handling: pad nibble ignored, row pitches honoured, sampled outputs.
# --------------------------------------------------------------------------
def test_odd_k_pad_nibble_is_never_read():
    rng = np.random.default_rng(11)
    M, K, N = 3, 2007, 13
    raw = _rand_codes(rng, N, K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    s = rng.uniform(0.005, 0.02, N).astype(np.float32)
    for order in ("low_first", "high_first"):
        a, _ = orc.linear(x, pack(raw, order, pad=0), s, None, K=K, group_size=0, order=order)
        b, _ = orc.linear(x, pack(raw, order, pad=15), s, None, K=K, group_size=0, order=order)
        assert np.array_equal(a, b)


def test_row_pitches_are_honoured():
    rng = np.random.default_rng(12)
    M, K, N, gs = 4, 130, 21, 32
    raw = _rand_codes(rng, N, K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    s = rng.uniform(0.005, 0.02, (-(-K // gs), N)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    a, da = orc.linear(x, pack(raw), s, bias, K=K, group_size=gs)
    xp = np.full((M, K + 7), np.nan, np.float32)
    xp[:, :K] = x
    qp = pack(raw, ldq=(K + 1) // 2 + 5)
    qp[:, (K + 1) // 2:] = 0xFF
    sp = np.full((s.shape[0], N + 3), np.nan, np.float32)
    sp[:, :N] = s
    b, db = orc.linear(xp, qp, sp, bias, K=K, group_size=gs)
    assert np.array_equal(a, b) and np.array_equal(da, db)


def test_sampled_outputs_match_full():
    rng = np.random.default_rng(13)
    M, K, N, gs = 6, 300, 70, 32
    qw = pack(_rand_codes(rng, N, K))
    x = rng.standard_normal((M, K)).astype(np.float32)
    s = rng.uniform(0.005, 0.02, (-(-K // gs), N)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    full, fden = orc.linear(x, qw, s, bias, K=K, group_size=gs)
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    out, den = orc.linear_sampled(x, qw, s, bias, ms, ns, K=K, group_size=gs)
    assert np.array_equal(out, full[ms, ns]) and np.array_equal(den, fden[ms, ns])


def test_thread_count_reported():
    assert orc.max_threads() >= 1
