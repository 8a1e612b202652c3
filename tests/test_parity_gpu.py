"""GPU parity: the HIP path against the fp64 oracle, element by element, on
seeded synthetic inputs at sizes the oracle finishes in seconds (several
tiles plus ragged tails), through the C ABI.

Shapes include the pages' own test shapes (page 1: steel M=96 K=2048 N=256,
steel_f16_edge M=70 K=1024 N=136, pwdq gs 64 and gs 8, the deep-K
128 x 8192 x 2048 case) and the decode GEMV of page 4 at reduced N.

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
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs, small_projection
from tests.gpu_util import check_case, log, need_gpu, run_gpu, oracle_full, normalised_error
from tests.packing import pack

pytestmark = pytest.mark.gpu


def inputs(M, K, N, gs, order="low_first", bias=False, seed=0, x_dist=("normal",)):
    p = small_projection(M, K, N, gs, order=order, has_bias=bias, x_dist=x_dist)
    return make_inputs(p, seed)


# ---- the tiny workload (M=4, K=256, N=128, gs 32, bias, seed 0) ----------
@pytest.mark.parametrize("math", ["auto", "f32", "f16"])
def test_tiny_config(math):
    need_gpu()
    p = CONFIGS["tiny"][0]
    x, qw, s, bias = make_inputs(p, 0)
    check_case(x, qw, s, bias, K=p.K, gs=p.group_size, order=p.order, math=math,
               label="tiny")


# ---- decode GEMV (M = 1) -------------------------------------------------
@pytest.mark.parametrize("K", [256, 300, 512, 1000, 2007, 2008, 2048, 4096, 8192, 14336,
                               20000])
@pytest.mark.parametrize("gs", [0, 32, 128])
def test_gemv_shapes(K, gs):
    need_gpu()
    N = 515
    if gs and K % gs and gs > K:
        gs = 32
    x, qw, s, bias = inputs(1, K, N, gs, bias=(K % 2 == 0), seed=K + gs)
    check_case(x, qw, s, bias, K=K, gs=gs, order="low_first", label="gemv")


@pytest.mark.parametrize("N", [1, 7, 8, 63, 257, 3000])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_gemv_ragged_n_and_order(N, order):
    need_gpu()
    x, qw, s, bias = inputs(1, 2008, N, 0, order=order, seed=N, x_dist=("uniform", -1, 1))
    check_case(x, qw, s, bias, K=2008, gs=0, order=order, label="gemv-ragged")


@pytest.mark.parametrize("gs", [8, 16, 24, 48, 100, 3])
def test_gemv_other_group_sizes(gs):
    need_gpu()
    x, qw, s, bias = inputs(1, 1000, 130, gs, bias=True, seed=gs)
    check_case(x, qw, s, bias, K=1000, gs=gs, order="low_first", label="gemv-gs")


@pytest.mark.parametrize("M", [2, 3, 5])
def test_f32_path_several_rows(M):
    need_gpu()
    x, qw, s, bias = inputs(M, 2048, 300, 32, bias=True, seed=M)
    check_case(x, qw, s, bias, K=2048, gs=32, order="low_first", math="f32", label="f32-M")


# ---- low batch: several activation rows per workgroup, fp32 --------------
@pytest.mark.parametrize("M,K,N,gs,order", [
    (2, 2048, 515, 32, "low_first"), (3, 256, 128, 32, "high_first"),
    (4, 8192, 700, 32, "low_first"), (5, 2008, 301, 0, "high_first"),
    (7, 2048, 1000, 0, "high_first"), (8, 4096, 257, 128, "low_first"),
    (9, 1024, 129, 64, "low_first"), (16, 2048, 300, 32, "high_first"),
    (6, 6000, 90, 32, "low_first"), (2, 20000, 64, 32, "low_first"),
    # four spans of 2048 k at M > 2: K split in two, four rows per workgroup
    (3, 8192, 301, 32, "high_first"), (16, 8192, 515, 32, "low_first"),
    (11, 6200, 260, 0, "low_first"), (4, 7000, 130, 64, "high_first"),
])
def test_lowbatch_f32(M, K, N, gs, order):
    """Weights read once for all M rows; held to the fp32 bar."""
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=(M % 2 == 0), seed=M * 100 + K)
    check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f32", label="lowbatch")


def test_lowbatch_pitches():
    need_gpu()
    x, qw, s, bias = inputs(4, 2048, 200, 32, bias=True, seed=41)
    check_case(x, qw, s, bias, K=2048, gs=32, order="low_first", math="f32",
               pad=(3, 4, 4, 5), label="lowbatch-pitch")


# ---- prefill GEMM (M > 1) ------------------------------------------------
@pytest.mark.parametrize("M,K,N,gs", [
    (96, 2048, 256, 32),     # page 1: steel
    (70, 1024, 136, 32),     # page 1: steel_f16_edge (partial M and N tiles)
    (96, 2048, 256, 64),     # page 1: pwdq_gs64
    (96, 2048, 256, 8),      # page 1: pwdq_gs8 (group smaller than the K slice)
    (128, 8192, 2048, 32),   # page 1: deep-K case
    (2, 256, 128, 32), (7, 2048, 1000, 0), (64, 2048, 512, 32), (65, 2008, 3000, 0),
    (130, 2007, 300, 32), (333, 2048, 700, 0), (256, 4096, 1024, 128),
    (17, 300, 77, 100), (40, 520, 64, 3), (513, 1024, 260, 16),
])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_gemm_shapes(M, K, N, gs, order):
    """The MFMA kernels at every shape (math forced to f16: for small batches
    the automatic choice is the fp32 low-batch GEMV, tested separately)."""
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=(M % 2 == 0), seed=M * 7 + N,
                            x_dist=("uniform", -1, 1))
    check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16", label="gemm")


@pytest.mark.parametrize("M,K,N,gs,expect", [
    (1, 2048, 300, 32, "gemv_f32"), (4, 2048, 300, 32, "gemv_f32"),
    (4, 2048, 2048, 32, "gemv_f32"), (2, 2048, 8192, 32, "gemv_f32"),
    (2, 8192, 2048, 32, "gemv_f32"), (3, 2048, 8192, 32, "gemm_f16_skinny"),
    (4, 2048, 8192, 32, "gemm_f16_skinny"), (8, 2048, 8192, 32, "gemm_f16_skinny"),
    (5, 2048, 2048, 32, "gemm_f16_skinny"), (16, 2048, 2048, 32, "gemm_f16_skinny"),
    (32, 2048, 300, 0, "gemm_f16_skinny"), (33, 2048, 300, 0, "gemm_f16_skinny"),
    (65, 2048, 300, 0, "gemm_f16_skinny"), (96, 2048, 4096, 128, "gemm_f16_skinny"),
    (97, 2048, 300, 0, "gemm_f16_skinny"), (256, 2048, 300, 0, "gemm_f16_skinny"),
    (1025, 2048, 300, 0, "gemm_f16"), (80, 2048, 8192, 32, "gemm_f16"),
    (128, 4096, 4096, 128, "gemm_f16_skinny"), (129, 4096, 4096, 128, "gemm_f16"),
    (65, 2008, 3000, 0, "gemm_f16_skinny"), (65, 2008, 3000, 32, "gemm_f16_skinny"),
    (65, 2010, 3000, 32, "gemm_f16"),
    (2, 2048, 128257, 0, "gemm_f16_skinny"), (7, 2048, 128257, 0, "gemm_f16_skinny"),
    (2, 14336, 4096, 128, "gemm_f16_skinny"), (3, 4096, 14336, 128, "gemm_f16_skinny"),
    (4, 2048, 300, 8, "gemm_f16"), (4, 2040, 300, 32, "gemv_f32"),
    (20, 2040, 300, 32, "gemm_f16_skinny"), (9, 2040, 2048, 32, "gemv_f32"),
])
def test_auto_regime(M, K, N, gs, expect):
    """The automatic choice of kernel, and its parity at that kernel's bar."""
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, bias=True, seed=M + N)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order="low_first", label="auto")
    assert path == expect


@pytest.mark.parametrize("math", ["f32", "f16"])
def test_row_pitches_and_unaligned_rows(math):
    need_gpu()
    M = 1 if math == "f32" else 33
    x, qw, s, bias = inputs(M, 1002, 200, 32, bias=True, seed=5)
    # ldq = 501 + 2 = 503 bytes: rows start at odd addresses
    check_case(x, qw, s, bias, K=1002, gs=32, order="low_first", math=math,
               pad=(5, 2, 3, 7), label="pitches")
    check_case(x, qw, s, bias, K=1002, gs=32, order="low_first", math=math,
               pad=(4, 3, 0, 1), label="pitches")


# ---- the pipelined GEMM's output stores ----------------------------------
# ---- the pipelined GEMM when K is not a multiple of its 64-k step ----------
# The binary16 pre-pass also copies each weight row's bytes of the last step
# (bytes past K as 0x88) and the kernel reads that step from the copy: even
# K of every remainder, rows of K / 2 bytes (K % 8 == 0) and padded to a
# dword, partial last groups, split K, 128 x 256 tiles.
@pytest.mark.parametrize("M,K,N,gs,qpad,order", [
    (1100, 2008, 3000, 0, 0, "high_first"),  # the 2008 x 3000 shape: K % 64 = 24
    (1100, 1000, 520, 32, 0, "low_first"),   # K % 64 = 40, a last group of 8
    (1100, 2040, 300, 128, 0, "high_first"), # a last group of 120
    (1100, 200, 3000, 0, 0, "low_first"),    # K % 64 = 8
    (96, 2010, 256, 32, 3, "low_first"),     # K % 8 = 2: rows of 1005 bytes padded to 1008
    (1100, 8200, 256, 32, 0, "high_first"),  # split K, the last step in the last split
    (136, 264, 16400, 32, 0, "low_first"),   # 128 x 256 tiles
])
def test_pipelined_gemm_k_tail(M, K, N, gs, qpad, order):
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=True, seed=M + K)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16",
                            pad=(0, qpad, 0, 0), label="pipe-ktail")
    assert path == "gemm_f16"


def test_pipelined_gemm_bytes_past_k_do_not_reach_the_sum():
    """Row bytes past K (the pitch's 0xFF padding: code 15) under scales of
    30000 would dequantize to inf in binary16, and inf * 0 = NaN; the last
    step's copy holds 0x88 there, so the result stays finite."""
    need_gpu()
    rng = np.random.default_rng(8)
    M, K, N = 1100, 2008, 300
    raw = rng.integers(7, 10, size=(N, K))  # c in {-1, 0, 1}: |c * s| <= 30000
    qw = torch.from_numpy(pack(raw, "low_first"))
    x = torch.from_numpy(rng.uniform(-1, 1, size=(M, K)).astype(np.float32))
    s = torch.full((N,), 30000.0)
    out, path, guards = run_gpu(x, qw, s, None, K=K, gs=0, order="low_first", math="f16",
                                pad=(0, 48, 0, 0))
    ref, den = oracle_full(x, qw, s, None, K=K, gs=0, order="low_first")
    assert path == "gemm_f16" and guards
    assert np.all(np.isfinite(out))
    assert normalised_error(out, ref, den) <= 2e-3


# The pipelined kernel (dword-aligned weight rows, even K, power-of-two
# groups >= 32 or per-channel) stores 16-byte row segments when the output
# rows allow it and element by element otherwise; split-K partials likewise.
# These shapes hit every branch: an output pitch that is not a multiple of 4,
# a last column quad that is partly past N, M tails, and split-K partials with
# N % 4 != 0, each with a bias and guard columns around the output.
@pytest.mark.parametrize("M,K,N,gs,pad_out", [
    (1100, 512, 203, 32, 3),    # no split; element stores (output pitch 206)
    (130, 2048, 8202, 64, 2),   # no split; 16-byte stores, last quad ragged, M tail
    (1100, 8192, 130, 128, 0),  # split K; element stores of partials (N % 4 == 2)
    (1100, 4096, 264, 32, 0),   # split K; 16-byte stores of partials
    (1100, 512, 516, 0, 0),     # per-channel scales; 16-byte stores, M tail
])
def test_pipelined_gemm_output_stores(M, K, N, gs, pad_out):
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, bias=True, seed=M + K + N)
    _, path, _ = check_case(x, qw, s, bias, K=K, gs=gs, order="low_first", math="f16",
                            pad=(0, 0, 0, pad_out), label="pipe-stores")
    assert path == "gemm_f16"


# ---- the pipelined GEMM's 128 x 256 tiles --------------------------------
# Without split-K, and where 128 x 128 tiles would number more than 256, the
# pipelined kernel runs 128 x 256 tiles (two 32-column blocks per wave, the
# tile leaving in two passes).  Each shape below has more than 256 narrow
# tiles and no split, a last wide tile that is partly past N, and an M tail.
@pytest.mark.parametrize("M,K,N,gs,order,pad_out", [
    (136, 256, 16400, 32, "low_first", 3),    # element stores (pitch 16403)
    (390, 256, 8300, 128, "high_first", 0),   # 16-byte stores, last quad whole
    (333, 256, 12290, 0, "low_first", 0),     # per-channel scales, last quad ragged
])
def test_pipelined_gemm_wide_tiles(M, K, N, gs, order, pad_out):
    need_gpu()
    x, qw, s, bias = inputs(M, K, N, gs, order=order, bias=True, seed=M + N)
    check_case(x, qw, s, bias, K=K, gs=gs, order=order, math="f16",
               pad=(0, 0, 0, pad_out), label="pipe-wide")


def test_pipelined_gemm_wide_tiles_binary16_scales():
    """q4f16_1 weights on the 128 x 256 tiles: the same values as fp32 scales
    holding the binary16 values, bit for bit, and within the MFMA bound of
    the oracle."""
    need_gpu()
    dev = torch.device("cuda")
    M, K, N = 300, 512, 11000
    x, qw, s, bias = inputs(M, K, N, 64, bias=True, seed=7)
    s16 = s.half()
    xd, qd, bd = x.to(dev), qw.to(dev), bias.to(dev)
    o16 = b.linear(xd, qd, s16.to(dev), bd, K=K, group_size=64, math="f16")
    o32 = b.linear(xd, qd, s16.float().to(dev), bd, K=K, group_size=64, math="f16")
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)
    ref, den = oracle_full(x, qw, s16.float(), bias, K=K, gs=64, order="low_first")
    err = normalised_error(o16.cpu().numpy(), ref, den)
    assert err <= 2e-3, err


@pytest.mark.parametrize("math,M,K,N", [
    ("f16", 130, 2048, 1030),   # pipelined GEMM, no split: the output's own stores
    ("f16", 64, 8192, 260),     # pipelined GEMM, split K: the reduce kernel's stores
    ("f16", 70, 1002, 300),     # general GEMM
    ("f32", 1, 2048, 515),      # GEMV
    ("f32", 4, 2048, 515),      # low-batch GEMV
])
def test_output_not_16_byte_aligned(math, M, K, N):
    """out may start at any 4-byte boundary: a view that begins one float
    into its buffer (so no 16-byte vector store is legal) gets the same
    values, and nothing outside [M, N] is written."""
    need_gpu()
    dev = torch.device("cuda")
    x, qw, s, bias = inputs(M, K, N, 32, bias=True, seed=M + N)
    obuf = torch.full((M + 2, N + 5), float("nan"), dtype=torch.float32, device=dev)
    out = obuf[:M, 1:N + 1]
    assert out.data_ptr() % 16 != 0
    b.linear(x.to(dev), qw.to(dev), s.to(dev), bias.to(dev), K=K, group_size=32, math=math,
             out=out)
    torch.cuda.synchronize()
    full = obuf.cpu().numpy()
    assert np.all(np.isnan(full[:, 0])) and np.all(np.isnan(full[:, N + 1:]))
    assert np.all(np.isnan(full[M:, :]))
    got = full[:M, 1:N + 1]
    ref, den = oracle_full(x, qw, s, bias, K=K, gs=32, order="low_first")
    err = normalised_error(got, ref, den)
    assert not np.any(np.isnan(got))
    assert err <= (2e-3 if math == "f16" else 1e-5), err


# ---- exact special cases (bit-for-bit on every path) ---------------------
@pytest.mark.parametrize("math,M", [("f32", 1), ("f32", 3), ("f16", 1), ("f16", 70),
                                    ("auto", 200)])
def test_integer_case_is_exact(math, M):
    """x in {-2..2} and scales 2^-6: every product and partial sum is exact in
    fp32 (and the operands exact in binary16), so all paths equal the oracle
    bit for bit, tails included."""
    need_gpu()
    rng = np.random.default_rng(M)
    K, N = 2008, 301
    raw = rng.integers(0, 16, size=(N, K))
    xi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    qw = torch.from_numpy(pack(raw, "high_first", pad=15))
    x = torch.from_numpy(xi)
    s = torch.full(((K + 31) // 32, N), 2.0 ** -6)
    bias = torch.from_numpy(rng.integers(-9, 10, size=N).astype(np.float32) * 2.0 ** -6)
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=32, order="high_first", math=math)
    ref, _ = oracle_full(x, qw, s, bias, K=K, gs=32, order="high_first")
    assert guards
    assert np.array_equal(out.astype(np.float64), ref), path


@pytest.mark.parametrize("math,M", [("auto", 1), ("auto", 9), ("f32", 4)])
def test_all_eights_give_the_bias(math, M):
    need_gpu()
    K, N = 777, 333
    x = torch.randn(M, K, generator=torch.Generator().manual_seed(3))
    qw = torch.full((N, (K + 1) // 2), 0x88, dtype=torch.uint8)
    s = torch.rand((K + 31) // 32, N, generator=torch.Generator().manual_seed(4))
    bias = torch.randn(N, generator=torch.Generator().manual_seed(5))
    out, path, guards = run_gpu(x, qw, s, bias, K=K, gs=32, order="low_first", math=math)
    assert guards
    assert np.array_equal(out, np.broadcast_to(bias.numpy(), (M, N))), path


def test_results_are_deterministic():
    need_gpu()
    for M, K, N in ((1, 8192, 2048), (1, 65536, 64), (512, 2048, 512)):
        x, qw, s, bias = inputs(M, K, N, 32, seed=11)
        a, _, _ = run_gpu(x, qw, s, bias, K=K, gs=32, order="low_first")
        c, _, _ = run_gpu(x, qw, s, bias, K=K, gs=32, order="low_first")
        assert np.array_equal(a, c)


# Split K in the pipelined GEMM: the splits' fp32 partials go through the
# workspace and the reduce kernel adds them in split order, then the bias.
# Repeated calls and graph replays (three kernels per call) must give the
# same bits, within the oracle's bound.
@pytest.mark.parametrize("M,K,N,gs,bias", [
    (513, 2048, 2048, 32, True),    # 80 tiles, 2 splits
    (512, 8192, 2048, 32, False),   # 64 tiles, 4 splits of 32 steps
    (1100, 8192, 130, 128, True),   # 18 tiles, 8 splits, N % 4 != 0 (element path)
    (1100, 4096, 600, 0, True),     # 45 tiles, 4 splits, ragged M and N
])
def test_pipelined_split_k_repeats_and_replays(M, K, N, gs, bias):
    need_gpu()
    x, qw, s, bv = inputs(M, K, N, gs, bias=bias, seed=M + N)
    dev = torch.device("cuda")
    xd, qd, sd = x.to(dev), qw.to(dev), s.to(dev)
    bd = bv.to(dev) if bias else None
    first, path = b.linear(xd, qd, sd, bd, K=K, group_size=gs, math="f16", return_path=True)
    torch.cuda.synchronize()
    assert path == "gemm_f16"
    ref, den = oracle_full(x, qw, s, bv if bias else None, K=K, gs=gs, order="low_first")
    assert normalised_error(first.cpu().numpy(), ref, den) <= 2e-3
    for _ in range(20):
        again = b.linear(xd, qd, sd, bd, K=K, group_size=gs, math="f16")
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))
    out = torch.empty(M, N, device=dev)
    ws = torch.empty(b.workspace_bytes(M, N, K, gs, "f16"), dtype=torch.uint8, device=dev)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        b.linear(xd, qd, sd, bd, K=K, group_size=gs, math="f16", out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        b.linear(xd, qd, sd, bd, K=K, group_size=gs, math="f16", out=out, workspace=ws)
    for _ in range(5):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), first.view(torch.int32))


def test_split_k_gemv_with_large_k():
    """K beyond one workgroup's cover forces the split-K plan and its
    reduce kernel."""
    need_gpu()
    x, qw, s, bias = inputs(1, 65536, 64, 32, bias=True, seed=2)
    check_case(x, qw, s, bias, K=65536, gs=32, order="low_first", label="gemv-splitk")


def test_empty_sizes_are_noops():
    need_gpu()
    from bit_weight_only_int4_amd import q4linear as b
    dev = torch.device("cuda")
    x = torch.empty(0, 64, device=dev)
    qw = torch.zeros(16, 32, dtype=torch.uint8, device=dev)
    s = torch.ones(2, 16, device=dev)
    out, path = b.linear(x, qw, s, group_size=32, return_path=True)
    assert out.shape == (0, 16) and path == "none"


@pytest.mark.parametrize("M,K,N,gs", [(64, 8192, 2048, 32), (1, 20480, 512, 32),
                                      (4, 8192, 1024, 32), (200, 1024, 640, 0)])
def test_workspace_16_byte_aligned(M, K, N, gs):
    """A workspace that is 16-byte but not 256-byte aligned is accepted and
    gives the same bits as the allocator's (256-byte aligned) one."""
    need_gpu()
    p = small_projection(M, K, N, gs)
    x, qw, s, bias = make_inputs(p, 7)
    dev = torch.device("cuda")
    xd, qd, sd = x.to(dev), qw.to(dev), s.to(dev)
    need = b.workspace_bytes(M, N, K, gs)
    assert need > 0
    ref = b.linear(xd, qd, sd, None, K=K, group_size=gs)
    buf = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws = buf[16:16 + need]
    assert ws.data_ptr() % 256 == 16
    out = b.linear(xd, qd, sd, None, K=K, group_size=gs, workspace=ws)
    torch.cuda.synchronize()
    log(f"[ws+16] M={M} K={K} N={N} gs={gs}")
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
