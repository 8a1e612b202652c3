"""GPU parity on seeded random shapes against the fp64 oracle, through the
C ABI: every kernel the automatic choice (or a forced math) picks, with
ragged M, N and K, group sizes of every kind, both nibble orders, row
pitches, bias on and off, NaN-poisoned outputs with guard rows and columns.
The shapes are drawn to fall around the kernels' boundaries: 1-4 rows (the
fp32 GEMVs), up to 32, 64 and 96 rows and beyond (the few-row kernel's row
blocks, up to 1024 rows on small weights), the tiled GEMM above, K a
multiple of 32, of 8, even or odd.
The bar is the path's own: 1e-5 for the fp32 GEMV, 2e-3 for binary16
operands, normalised by sum_k |x * w|.
"""
import numpy as np
import pytest

from bit_weight_only_int4_amd.workloads import make_inputs, small_projection
from tests.gpu_util import check_case, need_gpu

pytestmark = pytest.mark.gpu


def draw(i):
    rng = np.random.default_rng(1000 + i)
    M = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 31, 32, 33, 40, 48, 63, 64, 65,
                        70, 80, 95, 96, 97, 100, 128, 129, 200, 300, 512, 700]))
    kind = int(rng.integers(0, 4))
    if kind == 0:
        K = 32 * int(rng.integers(4, 130))       # whole 16-byte chunks
    elif kind == 1:
        K = 8 * int(rng.integers(16, 520))       # whole 8-k chunks
    elif kind == 2:
        K = 2 * int(rng.integers(40, 2100))      # even
    else:
        K = 2 * int(rng.integers(40, 2100)) + 1  # odd
    N = int(rng.integers(1, 3000))
    gs = int(rng.choice([0, 32, 64, 128, 256, 48, 16, 8, 100]))
    if gs > K:
        gs = 0
    while M * N * K > 1.5e8:
        N = max(1, N // 2)
    order = ["low_first", "high_first"][int(rng.integers(0, 2))]
    math = "auto" if rng.random() < 0.7 else ("f16" if M > 4 or rng.random() < 0.5 else "f32")
    pad = tuple(int(v) for v in rng.integers(0, 4, size=4)) if rng.random() < 0.3 else (0, 0, 0, 0)
    bias = bool(rng.random() < 0.5)
    return M, K, N, gs, order, math, pad, bias


@pytest.mark.parametrize("i", range(96))
def test_random_shape(i):
    need_gpu()
    M, K, N, gs, order, math, pad, bias = draw(i)
    p = small_projection(M, K, N, gs, order=order, has_bias=bias, x_dist=("uniform", -1, 1))
    x, qw, s, bv = make_inputs(p, i)
    check_case(x, qw, s, bv if bias else None, K=K, gs=gs, order=order, math=math, pad=pad,
               label=f"random-{i}")
