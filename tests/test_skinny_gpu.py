"""GPU parity of the few-row MFMA GEMM (M <= 1024) against the fp64 oracle,
through the C ABI, and the boundary between it and the tiled GEMM.

The kernel's plan depends on the sizes alone, so the shapes below are
chosen to reach each of its regimes (derived from the plan's rules, stated
beside each case):
  * waves of a workgroup along K (wk = 8, 4, 2) and along N only (wk = 1),
    the latter with several column blocks per persistent workgroup;
  * a K whose last 128-k step is partial (K % 128 != 0), and K % 32 != 0
    (whole 8-k chunks) where the scale is taken out of the sums;
  * K split across workgroups when one row block's binary16 activations
    exceed LDS (M = 16 and M = 32 at K = 8192), or when narrow N leaves CUs
    without a block (the down projections at few rows), with the split-K
    reduce;
  * staging of the activations in several rounds (M * K / 8 > 2048);
  * more than 32 rows: row blocks of 32 in separate workgroups (two to
    32);
  * ragged N, both nibble orders, per-channel and grouped scales (32, 128),
    fp32 and binary16 scales, bias on and off, row pitches, and a NaN-poisoned
    output with guard rows and columns.
The bar is the MFMA path's: max |gpu - ref| / sum_k |x * w| <= 2e-3.
"""
import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import make_inputs, small_projection
from tests.gpu_util import check_case, log, need_gpu, normalised_error, oracle_full, run_gpu
from tests.packing import pack

pytestmark = pytest.mark.gpu

SKINNY = "gemm_f16_skinny"


def inputs(M, K, N, gs, order="low_first", bias=False, seed=0):
    p = small_projection(M, K, N, gs, order=order, has_bias=bias, x_dist=("uniform", -1, 1))
    return make_inputs(p, seed)


@pytest.mark.parametrize("M", [1, 2, 4, 7, 16, 17, 24, 32, 33, 48, 64, 65, 96, 97, 128, 200,
                               257, 1024, 1025])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
@pytest.mark.parametrize("gs", [0, 32, 128])
def test_rows_around_the_boundary(M, order, gs):
    """M <= 1024 runs the skinny kernel here (M * N * K <= 2^31,
    N * K <= 2^24, N <= 4096; above 32 rows in row blocks of 32), M >= 1025
    the tiled GEMM;
    N = 1000 is ragged against 16- and 32-column blocks (wk = 8 here)."""
    need_gpu()
    K, N = 2048, 1000
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=(M % 2 == 1), seed=M * 31 + gs)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16",
                            label="skinny-boundary")
    assert path == (SKINNY if M <= 1024 else "gemm_f16")


@pytest.mark.parametrize("M,K,N,gs,expect", [
    (40, 4096, 14336, 128, "gemm_f16"),      # N * K > 2^25: the tiled GEMM
    (33, 2048, 16384, 32, SKINNY),           # N * K = 2^25
    (33, 2048, 16385, 32, "gemm_f16"),
    (50, 2048, 70000, 0, SKINNY),            # vocabulary-sized N
    (64, 8192, 2048, 32, SKINNY),            # two row blocks, K split over 4 + reduce
    (41, 256, 3000, 32, SKINNY),             # two row blocks, the second of 9 rows
    (65, 2048, 4096, 128, SKINNY),           # three row blocks, the third of 1 row
    (90, 8192, 2048, 32, SKINNY),            # three row blocks, K split over 4 + reduce
    (96, 4096, 4096, 0, SKINNY),             # N * K = 2^24, N = 4096
    (70, 2048, 4097, 0, "gemm_f16"),         # N > 4096 above 64 rows: the tiled GEMM
    (140, 4104, 4096, 0, "gemm_f16"),        # M * N * K > 2^31
    (128, 4096, 4096, 0, SKINNY),            # four row blocks, N * K = 2^24
    (129, 4096, 4096, 0, "gemm_f16"),        # M * N * K > 2^31
    (36, 14336, 4096, 128, "gemm_f16"),      # N * K > 2^25 above 32 rows
    (512, 2048, 2048, 32, SKINNY),           # 16 row blocks, M * N * K = 2^31
    (513, 2048, 2048, 32, "gemm_f16"),
    (256, 2048, 4096, 128, SKINNY),          # eight row blocks, N * K = 2^23
    (250, 8192, 1000, 32, SKINNY),           # eight row blocks, the last of 26 rows, K split
])
def test_row_blocks(M, K, N, gs, expect):
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, bias=True, seed=M + K + N)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order="high_first", math="f16",
                            label="skinny-rows")
    assert path == expect


@pytest.mark.parametrize("M,K,N,gs,note", [
    (3, 256, 140000, 32, "wk=1, 547 blocks over 512 workgroups: two blocks on some"),
    (5, 256, 40000, 0, "wk=2"),
    (9, 2048, 20000, 128, "wk=4"),
    (7, 2080, 300, 32, "K % 128 = 32: partial last step, wk=8 with spw=3 > 17/8"),
    (20, 160, 77, 32, "two steps, the second partial; wk=2"),
    (32, 2048, 256, 32, "activations staged in four rounds"),
    (16, 8192, 300, 32, "K split over 2 workgroups + reduce"),
    (32, 8192, 520, 128, "K split over 4 workgroups + reduce, 160 KiB of LDS"),
    (4, 8192, 2048, 32, "the 1B down projection at M=4: K split over 4 workgroups for parallelism"),
    (2, 14336, 4096, 128, "the 8B down projection at M=2: K split over 2 for parallelism"),
    (16, 4096, 4096, 128, "16 rows, 4 steps a wave: K split over 2 for parallelism"),
    (8, 4096, 4096, 128, "8 rows, 4 steps a wave: one slice"),
    (7, 2048, 8192, 0, "the 1B gate projection, per-channel"),
    (1, 4096, 777, 32, "one row"),
    (12, 128, 33, 32, "the smallest K"),
])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_plan_regimes(M, K, N, gs, note, order):
    need_gpu()
    log(f"[skinny] {note}")
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=(N % 2 == 0), seed=M + K + N)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16",
                            label="skinny-plan")
    assert path == SKINNY


@pytest.mark.parametrize("pad", [(5, 4, 3, 7), (1, 0, 2, 1), (0, 8, 0, 3)])
def test_row_pitches(pad):
    """x, scale and output pitches; dword-aligned weight pitches stay on the
    skinny kernel."""
    need_gpu()
    x, qw, s, bias = inputs(11, 2048, 333, 32, bias=True, seed=17)
    _, path, _ = check_case(x, qw, s, bias, K=2048, gs=32, order="low_first", math="f16",
                            pad=pad, label="skinny-pitch")
    assert path == SKINNY


def test_unaligned_weight_rows_take_the_tiled_kernel():
    need_gpu()
    x, qw, s, bias = inputs(11, 2048, 333, 32, bias=True, seed=18)
    _, path, _ = check_case(x, qw, s, bias, K=2048, gs=32, order="low_first", math="f16",
                            pad=(0, 1, 0, 0), label="skinny-unaligned")
    assert path == "gemm_f16"


@pytest.mark.parametrize("M,K,gs", [(8, 2056, 32), (8, 2056, 64), (8, 2048, 64), (8, 2048, 48),
                                    (8, 2048, 16), (8, 2052, 0)])
def test_other_shapes_take_the_tiled_kernel(M, K, gs):
    """K % 8 != 0 and groups that are not powers of two >= 32 are the
    tiled kernel's; K % 32 != 0 with groups of 32 or 64 stays on the few-row
    kernel (a zero scale for the words past K)."""
    need_gpu()
    x, qw, s, bias = inputs(M, K, 200, gs, seed=19)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order="low_first", math="f16",
                            label="skinny-other")
    assert path == (SKINNY if (gs in (32, 64) and K % 8 == 0) else "gemm_f16")


@pytest.mark.parametrize("M,gs", [(7, 0), (24, 32), (5, 128)])
def test_binary16_scales(M, gs):
    """q4f16_1 weights: binary16 scales give the same operands (a binary16
    scale is its own RN16), hence the same bits as their fp32 widening."""
    need_gpu()
    K, N = 2048, 600
    x, qw, s, bias = inputs(M, K, N, gs, bias=True, seed=23)
    dev = torch.device("cuda")
    s16 = s.half()
    xd, qd, bd = x.to(dev), qw.to(dev), bias.to(dev)
    o16, p16 = b.linear(xd, qd, s16.to(dev), bd, K=K, group_size=gs, math="f16",
                        return_path=True)
    o32, p32 = b.linear(xd, qd, s16.float().to(dev), bd, K=K, group_size=gs, math="f16",
                        return_path=True)
    torch.cuda.synchronize()
    assert p16 == p32 == SKINNY
    assert torch.equal(o16.view(torch.int32), o32.view(torch.int32))
    ref, den = oracle_full(x, qw, s16.float(), bias, K=K, gs=gs, order="low_first")
    assert normalised_error(o16.cpu().numpy(), ref, den) <= 2e-3


@pytest.mark.parametrize("M", [1, 7, 16, 32, 48, 64])
def test_integer_case_is_exact(M):
    """x in {-2..2}, scales 2^-6: every operand is exact in binary16 and every
    partial sum exact in fp32, so the kernel equals the oracle bit for bit
    (K % 128 != 0: the partial last step included)."""
    need_gpu()
    rng = np.random.default_rng(100 + M)
    K, N = 2080, 301
    raw = rng.integers(0, 16, size=(N, K))
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    qw = torch.from_numpy(pack(raw, "high_first"))
    s = torch.full((K // 32, N), 2.0 ** -6)
    bias = torch.from_numpy(rng.integers(-9, 10, size=N).astype(np.float32) * 2.0 ** -6)
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=32, order="high_first", math="f16")
    ref, _ = oracle_full(x, qw, s, bias, K=K, gs=32, order="high_first")
    assert path == SKINNY and guards
    assert np.array_equal(out.astype(np.float64), ref)


def test_bytes_past_k_do_not_reach_the_sum():
    """The last 128-k step reads whole 16-byte chunks; those past K hold the
    row pitch's padding (0xFF: code 15).  With scales of 30000 such a code
    would dequantize to +inf in binary16, and inf * 0 = NaN; the kernel
    replaces the words past K by code 8 (c = 0), so the result stays finite
    and matches the oracle."""
    need_gpu()
    rng = np.random.default_rng(7)
    M, K, N = 5, 2080, 100
    raw = rng.integers(7, 10, size=(N, K))  # c in {-1, 0, 1}: |c * s| <= 30000
    qw = torch.from_numpy(pack(raw, "low_first"))
    x = torch.from_numpy(rng.uniform(-1, 1, size=(M, K)).astype(np.float32))
    s = torch.full((K // 32, N), 30000.0)
    out, path, guards = run_gpu(x, qw, s, None, K=K, gs=32, order="low_first", math="f16",
                                pad=(0, 48, 0, 0))
    ref, den = oracle_full(x, qw, s, None, K=K, gs=32, order="low_first")
    assert path == SKINNY and guards
    assert np.all(np.isfinite(out))
    assert normalised_error(out, ref, den) <= 2e-3


def test_all_eights_give_the_bias():
    need_gpu()
    M, K, N = 9, 1024, 333
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(3))
    qw = torch.full((N, K // 2), 0x88, dtype=torch.uint8)
    s = torch.rand(K // 32, N, generator=torch.Generator().manual_seed(4))
    bias = torch.randn(N, generator=torch.Generator().manual_seed(5))
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=32, order="low_first", math="f16")
    assert path == SKINNY and guards
    assert np.array_equal(out, np.broadcast_to(bias.numpy(), (M, N)))


def test_repeat_calls_are_bit_identical():
    need_gpu()
    for M, K, N, gs in ((7, 2048, 3000, 0), (32, 8192, 520, 128), (4, 256, 70000, 32)):
        x, qw, s, bias = inputs(M, K, N, gs, bias=True, seed=29)
        a, pa, _ = run_gpu(x, qw, s, bias, K=K, gs=gs, order="low_first", math="f16")
        c, pc, _ = run_gpu(x, qw, s, bias, K=K, gs=gs, order="low_first", math="f16")
        assert pa == pc == SKINNY
        assert np.array_equal(a, c)


# ---- K % 32 != 0: whole 8-k chunks, the scale taken out of the sums -------
# The last 16-byte weight chunk of a row then reaches past K: its bytes past
# the row belong to the row pitch, the next row or (last row) lie past the
# array, where the buffer load returns zeros.  They decode to finite codes
# (B = c exactly, no scale in the operand) and meet activations that the
# staging set to zero past K, so they add exactly nothing.
@pytest.mark.parametrize("M,K,N,gs,order", [
    (65, 2008, 3000, 0, "high_first"),   # the 2008 x 3000 workload, three row blocks
    (7, 2008, 300, 128, "low_first"),    # a last group of 88
    (33, 1000, 513, 0, "low_first"),     # K % 128 = 104, two row blocks
    (5, 2056, 200, 0, "high_first"),     # K % 32 = 8
    (96, 2040, 3000, 128, "low_first"),  # K % 32 = 24, three row blocks
    (16, 8200, 300, 0, "high_first"),    # K split over workgroups, the straddle in the last slice
    (3, 136, 70, 0, "low_first"),        # two steps, the second of 8 k
    (300, 2008, 3000, 0, "low_first"),   # ten row blocks, the last of 12 rows
    (7, 2008, 300, 32, "high_first"),    # groups of 32: the straddling chunk's last
                                         # word past K gets a zero scale
    (33, 1000, 513, 64, "low_first"),    # groups of 64, a last group of 40
    (5, 2056, 200, 32, "low_first"),     # K % 32 = 8: three words of the chunk past K
    (96, 2040, 3000, 32, "high_first"),  # K % 32 = 24, three row blocks
    (16, 8200, 300, 32, "low_first"),    # K split over workgroups
    (700, 1000, 2000, 128, "high_first"),  # 22 row blocks, groups of 128
])
def test_k_not_a_multiple_of_32(M, K, N, gs, order):
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=(M % 2 == 1), seed=M + K + N)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16",
                            label="skinny-k8")
    assert path == SKINNY


@pytest.mark.parametrize("M,gs", [(5, 0), (40, 128), (7, 32), (33, 64)])
def test_k_not_a_multiple_of_32_bytes_past_k(M, gs):
    """Row pitch padding of 0xFF (code 15) past K = 2008 and scales of 30000:
    the straddling chunk's bytes past K still add nothing, and nothing turns
    into inf or NaN."""
    need_gpu()
    rng = np.random.default_rng(11 + M)
    K, N = 2008, 300
    raw = rng.integers(7, 10, size=(N, K))
    qw = torch.from_numpy(pack(raw, "low_first"))
    x = torch.from_numpy(rng.uniform(-1, 1, size=(M, K)).astype(np.float32))
    s = torch.full((N,) if gs == 0 else ((K + gs - 1) // gs, N), 30000.0)
    out, path, guards = run_gpu(x, qw, s, None, K=K, gs=gs, order="low_first", math="f16",
                                pad=(0, 48, 0, 0))
    ref, den = oracle_full(x, qw, s, None, K=K, gs=gs, order="low_first")
    assert path == SKINNY and guards
    assert np.all(np.isfinite(out))
    assert normalised_error(out, ref, den) <= 2e-3


@pytest.mark.parametrize("M", [1, 33, 65])
def test_k_not_a_multiple_of_32_integer_case_is_exact(M):
    """x in {-2..2}, per-channel scales 2^-6, K = 2008: exact operands and
    partial sums, so the kernel equals the oracle bit for bit."""
    need_gpu()
    rng = np.random.default_rng(200 + M)
    K, N = 2008, 301
    raw = rng.integers(0, 16, size=(N, K))
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    qw = torch.from_numpy(pack(raw, "high_first"))
    s = torch.full((N,), 2.0 ** -6)
    out, path, guards = run_gpu(x, qw, s, None, K=K, gs=0, order="high_first", math="f16")
    ref, _ = oracle_full(x, qw, s, None, K=K, gs=0, order="high_first")
    assert path == SKINNY and guards
    assert np.array_equal(out.astype(np.float64), ref)
