"""GPU parity of the streaming GEMV's integer inner products against the
fp64 oracle, through the C ABI.

One activation row with K <= 2048 and N * K >= 2^27 (the output head) runs
the streaming GEMV on integer inner products: each lane's 32-k activation
chunk is written as block fixed point (27 significant bits against the
chunk's largest |x|) and sum_k c_k X_k is formed exactly in int32 by
v_dot8_i32_i4, with one fp32 rounding per chunk.  The cases aim at where
that differs from a per-element fp32 sum:
  * one outlier per chunk, 1e4 times the rest: the small values keep about
    13 bits against it, and the error against sum_k |x * w| stays orders
    below the bar;
  * values spread over many binades, down to fp32 subnormals;
  * the integer special case, exact (x_k 2^(26 - E) is an integer);
  * all codes 8: every sum is exactly zero and the bias comes out as is;
  * an inf or a NaN activation: every output is non-finite;
  * both nibble orders, per-channel and grouped (32, 128) scales, bias.
The bar is the fp32 path's: max |gpu - ref| / sum_k |x * w| <= 1e-5.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import check_case, log, need_gpu, oracle_full, run_gpu
from tests.packing import pack

pytestmark = pytest.mark.gpu

K = 2048
N = 65600  # N * K >= 2^27: the streaming kernel, one span


def weights(gs, order, seed):
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 16, size=(N, K))
    qw = torch.from_numpy(pack(raw, order))
    shape = (N,) if gs == 0 else (K // gs, N)
    s = torch.from_numpy(rng.uniform(0.005, 0.02, size=shape).astype(np.float32))
    return qw, s


@pytest.mark.parametrize("order", ["low_first", "high_first"])
@pytest.mark.parametrize("gs", [0, 32, 128])
def test_one_outlier_per_chunk(order, gs):
    need_gpu()
    rng = np.random.default_rng(gs + (order == "high_first"))
    x = rng.standard_normal((1, K)).astype(np.float32)
    pos = np.arange(0, K, 32) + rng.integers(0, 32, size=K // 32)
    x[0, pos] *= 1e4
    qw, s = weights(gs, order, 5 + gs)
    bias = torch.from_numpy(rng.uniform(-0.1, 0.1, N).astype(np.float32)) if gs == 32 else None
    _, path, err = check_case(torch.from_numpy(x), qw, s, bias, K=K, gs=gs, order=order,
                              label="digits-outlier")
    assert path == "gemv_f32"


def test_values_over_many_binades():
    """|x| from 1e-40 (fp32 subnormals) to 1e3, log-uniform, random signs."""
    need_gpu()
    rng = np.random.default_rng(9)
    mag = 10.0 ** rng.uniform(-40, 3, size=K)
    x = (mag * rng.choice([-1.0, 1.0], size=K)).astype(np.float32)[None, :]
    qw, s = weights(32, "low_first", 6)
    check_case(torch.from_numpy(x), qw, s, None, K=K, gs=32, order="low_first",
               label="digits-binades")


def test_integer_case_is_exact():
    need_gpu()
    rng = np.random.default_rng(12)
    raw = rng.integers(0, 16, size=(N, K))
    qw = torch.from_numpy(pack(raw, "high_first"))
    x = torch.from_numpy(rng.integers(-2, 3, size=(1, K)).astype(np.float32))
    s = torch.full((K // 32, N), 2.0 ** -6)
    bias = torch.from_numpy(rng.integers(-9, 10, size=N).astype(np.float32) * 2.0 ** -6)
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=32, order="high_first")
    ref, _ = oracle_full(x, qw, s, bias, K=K, gs=32, order="high_first")
    assert guards and path == "gemv_f32"
    assert np.array_equal(out.astype(np.float64), ref)


def test_all_eights_give_the_bias():
    need_gpu()
    x = torch.randn(1, K, generator=torch.Generator().manual_seed(3))
    qw = torch.full((N, K // 2), 0x88, dtype=torch.uint8)
    s = torch.rand(N, generator=torch.Generator().manual_seed(4)) + 0.5
    bias = torch.randn(N, generator=torch.Generator().manual_seed(5))
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=0, order="low_first")
    assert guards and path == "gemv_f32"
    assert np.array_equal(out, np.broadcast_to(bias.numpy(), (1, N)))


@pytest.mark.parametrize("bad", [float("inf"), float("-inf"), float("nan")])
def test_non_finite_activation_reaches_every_output(bad):
    need_gpu()
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, K)).astype(np.float32)
    x[0, 777] = bad
    qw, s = weights(0, "low_first", 8)
    # output buffer zero-filled (not NaN-poisoned), so that a row left
    # unwritten would show as finite
    out, path, _ = run_gpu(torch.from_numpy(x), qw, s, None, K=K, gs=0, order="low_first",
                           poison=False)
    ref, _ = oracle_full(torch.from_numpy(x), qw, s, None, K=K, gs=0, order="low_first")
    log(f"[digits] x[777] = {bad}: non-finite outputs {np.sum(~np.isfinite(out))} of {N}")
    assert path == "gemv_f32"
    assert not np.any(np.isfinite(ref))
    assert not np.any(np.isfinite(out))
