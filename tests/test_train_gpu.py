"""GPU parity of the training-side entry points against the oracle.

  * q4_requant: the packed codes are bit-identical to the oracle's
    (clamp(round(latent / s), -8, 7) + 8, ties to even, zero scale -> 8), on
    latents that mix in-range values, exact ties, clamped magnitudes, zero
    scales, infinities and NaN; bytes past ceil(K/2) stay untouched.
  * q4_linear_backward: dx = dout . dequant(W) within 1e-5 (fp32 path) or
    2e-3 (binary16 operands on MFMA) of the fp64 oracle, normalised by
    sum_n |dout * w| (exact where that is 0), with NaN-poisoned outputs,
    guard slots and padded pitches.
Page 3, "Add fp32 matmul ops (mm, bmm, linear)", stack entries #20943,
#20945 and #20946.
"""
import zlib

import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import CONFIGS
from oracle import q4_oracle as orc
from tests.gpu_util import log, need_gpu, normalised_error
from tests.packing import pack

pytestmark = pytest.mark.gpu

# fp32 path; binary16 operands on MFMA with fp32 sums (the forward's bars)
BWD_TOL = {"bwd_f32": 1e-5, "bwd_f16": 2e-3}


def _scales(rng, N, K, gs, lo=0.005, hi=0.02):
    shape = (N,) if gs == 0 else (-(-K // gs), N)
    return rng.uniform(lo, hi, shape).astype(np.float32)


def _latent(rng, N, K, scales, gs):
    """Latent weights: mostly in range, with exact ties, clamped values and
    a sprinkle of infinities and NaN."""
    S = scales[None, :].repeat(K, 0).T if gs == 0 else scales[np.arange(K) // gs][:, :N].T
    base = rng.standard_normal((N, K)) * 4.0
    ties = np.floor(rng.uniform(-9, 8, (N, K))) + 0.5
    pick = rng.uniform(0, 1, (N, K))
    q = np.where(pick < 0.15, ties, base)
    q = np.where(pick > 0.97, q * 50.0, q)
    lat = (q * S).astype(np.float32)
    flat = lat.reshape(-1)
    idx = rng.integers(0, flat.size, max(1, flat.size // 5000))
    flat[idx[0::3]] = np.inf
    flat[idx[1::3]] = -np.inf
    flat[idx[2::3]] = np.nan
    return lat


def _requant_case(N, K, gs, order, *, pad=0, zero_cols=0, seed=0):
    log(f"[requant] N={N} K={K} gs={gs} order={order} pad={pad}")
    rng = np.random.default_rng(seed)
    scales = _scales(rng, N, K, gs)
    if zero_cols:
        cols = rng.choice(N, zero_cols, replace=False)
        if gs == 0:
            scales[cols] = 0.0
        else:
            scales[0, cols] = 0.0
    latent = _latent(rng, N, K, scales, gs)
    Kp = (K + 1) // 2
    want = orc.requant(latent, scales, group_size=gs, order=order, ldq=Kp + pad, fill=0xAB)
    dev = torch.device("cuda")
    qbuf = torch.full((N, Kp + pad), 0xAB, dtype=torch.uint8, device=dev)
    got = b.requant(torch.from_numpy(latent).to(dev), torch.from_numpy(scales).to(dev),
                    group_size=gs, nibble_order=order, qw=qbuf[:, :Kp])
    torch.cuda.synchronize()
    assert got.data_ptr() == qbuf.data_ptr()
    assert np.array_equal(qbuf.cpu().numpy(), want)


@pytest.mark.parametrize("N,K,gs,order,pad", [
    (37, 256, 32, "low_first", 0), (33, 2008, 0, "high_first", 3),
    (17, 1001, 8, "low_first", 1), (5, 7, 3, "high_first", 0),
    (64, 4096, 128, "low_first", 4), (9, 67, 16, "high_first", 2),
    (3, 1, 0, "low_first", 0), (130, 513, 100, "low_first", 0)])
def test_requant_bit_exact(N, K, gs, order, pad):
    need_gpu()
    _requant_case(N, K, gs, order, pad=pad, zero_cols=min(3, N), seed=N * 131 + K)


@pytest.mark.parametrize("name", ["decode_1b", "llama8b_gs128", "per_channel_edges"])
def test_requant_full_size(name):
    """The largest weight of each workload, bit-exact over every byte."""
    need_gpu()
    p = max(CONFIGS[name], key=lambda q: q.N * q.K)
    _requant_case(p.N, p.K, p.group_size, p.order, seed=zlib.crc32(name.encode()))


def test_requant_round_trip_through_dequant():
    """requant(dequant_f32(q)) == q on the GPU, both orders."""
    need_gpu()
    rng = np.random.default_rng(5)
    dev = torch.device("cuda")
    for order in ("low_first", "high_first"):
        N, K, gs = 96, 1000, 32
        raw = rng.integers(0, 16, (N, K))
        qw = pack(raw, order, pad=8)
        scales = _scales(rng, N, K, gs)
        w = b.dequant(torch.from_numpy(qw).to(dev), torch.from_numpy(scales).to(dev), K, gs,
                      order, torch.float32)
        back = b.requant(w, torch.from_numpy(scales).to(dev), group_size=gs, nibble_order=order)
        assert np.array_equal(back.cpu().numpy(), qw)


def _bwd_case(M, N, K, gs, order, *, pad=(0, 0, 0, 0), seed=0, all_eights=False,
              math="auto"):
    log(f"[backward] M={M} N={N} K={K} gs={gs} order={order} pad={pad} math={math}")
    rng = np.random.default_rng(seed)
    raw = np.full((N, K), 8) if all_eights else rng.integers(0, 16, (N, K))
    qw = pack(raw, order, pad=int(rng.integers(0, 16)))
    scales = _scales(rng, N, K, gs)
    dout = rng.standard_normal((M, N)).astype(np.float32)
    ref, den = orc.linear_backward(dout, qw, scales, K=K, group_size=gs, order=order)
    dev = torch.device("cuda")

    def padded(a, extra, fill):
        t = torch.from_numpy(a)
        if t.dim() == 1 or extra == 0:
            return t.to(dev).contiguous()
        buf = torch.full((t.shape[0], t.shape[1] + extra), fill, dtype=t.dtype, device=dev)
        buf[:, : t.shape[1]] = t.to(dev)
        return buf[:, : t.shape[1]]

    dd = padded(dout, pad[0], float("nan"))
    qd = padded(qw, pad[1], 0xFF)
    sd = padded(scales, pad[2], float("nan"))
    dbuf = torch.full((M + 2, K + pad[3]), float("nan"), dtype=torch.float32, device=dev)
    dx = dbuf[:M, :K]
    _, path = b.linear_backward(dd, qd, sd, K=K, group_size=gs, nibble_order=order, dx=dx,
                                math=math, return_path=True)
    torch.cuda.synchronize()
    full = dbuf.cpu().numpy()
    auto_f16 = M >= 16 and (gs == 0 or gs >= K or gs % 8 == 0)
    assert path == ("bwd_f16" if math == "f16" or (math == "auto" and auto_f16) else "bwd_f32")
    tol = BWD_TOL[path]
    assert np.all(np.isnan(full[M:, :])) and np.all(np.isnan(full[:M, K:])), "guard written"
    got = full[:M, :K]
    assert not np.any(np.isnan(got))
    err = normalised_error(got, ref, den)
    log(f"          path={path} max normalised error={err:.3e} (tol {tol:.0e})")
    assert err <= tol
    return got


@pytest.mark.parametrize("M,N,K,gs,order,pad", [
    (1, 515, 2048, 32, "low_first", (0, 0, 0, 0)),
    (1, 8192, 2048, 32, "low_first", (0, 0, 0, 0)),
    (1, 2048, 8192, 32, "high_first", (3, 4, 1, 5)),
    (2, 300, 1000, 8, "high_first", (0, 0, 0, 0)),
    (3, 129, 67, 3, "low_first", (1, 2, 3, 4)),
    (4, 2048, 8192, 32, "low_first", (0, 0, 0, 0)),
    (7, 1000, 2008, 0, "high_first", (0, 1, 0, 0)),
    (16, 640, 512, 128, "low_first", (0, 0, 0, 0)),
    (33, 256, 300, 100, "low_first", (0, 0, 0, 0)),
    (1, 3, 1, 0, "low_first", (0, 0, 0, 0)),
    # dword-aligned rows with K % 32 == 0 at one to three rows: per-channel,
    # groups of 32 / 128 / 96 and 8 / 24; K past the last 512-k block; ragged
    # N; several row blocks (partial sums and the reduce)
    (1, 515, 2080, 0, "high_first", (0, 0, 0, 0)),
    (2, 700, 1024, 96, "low_first", (2, 4, 1, 3)),
    (2, 333, 4096, 128, "high_first", (0, 8, 0, 0)),
    (3, 1000, 2048, 8, "low_first", (0, 0, 0, 0)),
    (1, 4097, 512, 24, "high_first", (1, 0, 2, 0)),
    (2, 64, 160, 32, "low_first", (0, 0, 0, 0)),
])
def test_backward_parity(M, N, K, gs, order, pad):
    need_gpu()
    _bwd_case(M, N, K, gs, order, pad=pad, seed=M * 1000 + N + K)


def test_backward_prefill_sized_sampled():
    """M = 512 over a 1B-shaped weight on the fp32 path, checked on sampled
    elements."""
    need_gpu()
    rng = np.random.default_rng(512)
    M, N, K, gs = 512, 2048, 2048, 32
    qw = pack(rng.integers(0, 16, (N, K)))
    scales = _scales(rng, N, K, gs)
    dout = rng.standard_normal((M, N)).astype(np.float32)
    dev = torch.device("cuda")
    got = b.linear_backward(torch.from_numpy(dout).to(dev), torch.from_numpy(qw).to(dev),
                            torch.from_numpy(scales).to(dev), K=K, group_size=gs, math="f32")
    torch.cuda.synchronize()
    ms = rng.integers(0, M, 400)
    ks = rng.integers(0, K, 400)
    ref, den = orc.linear_backward_sampled(dout, qw, scales, ms, ks, K=K, group_size=gs)
    err = normalised_error(got.cpu().numpy()[ms, ks], ref, den)
    log(f"[backward M=512] max normalised error={err:.3e}")
    assert err <= 1e-5


def test_backward_all_eights_is_exactly_zero():
    need_gpu()
    got = _bwd_case(3, 700, 1024, 32, "low_first", seed=3, all_eights=True)
    assert np.all(got == 0)


def test_backward_is_deterministic():
    need_gpu()
    rng = np.random.default_rng(9)
    M, N, K, gs = 2, 4096, 2048, 32
    dev = torch.device("cuda")
    qw = torch.from_numpy(pack(rng.integers(0, 16, (N, K)))).to(dev)
    scales = torch.from_numpy(_scales(rng, N, K, gs)).to(dev)
    dout = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
    a = b.linear_backward(dout, qw, scales, K=K, group_size=gs)
    c = b.linear_backward(dout, qw, scales, K=K, group_size=gs)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("name", ["decode_1b", "llama8b_gs128", "per_channel_edges"])
def test_backward_full_size_sampled(name):
    """Every weight of a workload at full size, M = 1, on 300 sampled
    gradient elements computed one by one by the oracle."""
    need_gpu()
    from bit_weight_only_int4_amd.workloads import make_inputs
    dev = torch.device("cuda")
    for p in CONFIGS[name]:
        if p.M != 1:
            continue
        seed = zlib.crc32(p.name.encode())
        log(f"[backward full] {p.name} seed={seed}")
        _, qw, scales, _ = make_inputs(p, seed)
        g = torch.Generator().manual_seed(seed + 1)
        dout = torch.randn((1, p.N), generator=g)
        got = b.linear_backward(dout.to(dev), qw.to(dev), scales.to(dev), K=p.K,
                                group_size=p.group_size, nibble_order=p.order)
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed)
        ks = rng.integers(0, p.K, 300)
        ms = np.zeros(300, dtype=np.int64)
        ref, den = orc.linear_backward_sampled(dout.numpy(), qw.numpy(), scales.numpy(), ms, ks,
                                               K=p.K, group_size=p.group_size, order=p.order)
        err = normalised_error(got.cpu().numpy()[0, ks], ref, den)
        log(f"          max normalised error={err:.3e}")
        assert err <= 1e-5


# ---- the MFMA input gradient (math="f16") ---------------------------------
@pytest.mark.parametrize("M,N,K,gs,order,pad", [
    (1, 515, 2048, 32, "low_first", (0, 0, 0, 0)),
    (2, 300, 1000, 8, "high_first", (0, 0, 0, 0)),
    (33, 256, 300, 24, "low_first", (1, 2, 3, 4)),
    (128, 2048, 512, 128, "high_first", (0, 0, 0, 0)),
    (130, 1000, 2008, 0, "high_first", (0, 1, 0, 0)),
    (70, 4096, 1024, 32, "low_first", (0, 0, 0, 0)),
    (257, 640, 2007, 32, "low_first", (3, 4, 1, 5)),
    (64, 77, 129, 16, "high_first", (0, 3, 0, 0)),
    (5, 3, 1, 0, "low_first", (0, 0, 0, 0)),
])
def test_backward_f16_parity(M, N, K, gs, order, pad):
    need_gpu()
    _bwd_case(M, N, K, gs, order, pad=pad, seed=M * 977 + N + K, math="f16")


def test_backward_f16_all_eights_and_determinism():
    need_gpu()
    got = _bwd_case(40, 700, 1024, 32, "low_first", seed=4, all_eights=True, math="f16")
    assert np.all(got == 0)
    rng = np.random.default_rng(10)
    M, N, K, gs = 96, 4096, 2048, 32
    dev = torch.device("cuda")
    qw = torch.from_numpy(pack(rng.integers(0, 16, (N, K)))).to(dev)
    scales = torch.from_numpy(_scales(rng, N, K, gs)).to(dev)
    dout = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
    a = b.linear_backward(dout, qw, scales, K=K, group_size=gs, math="f16")
    c = b.linear_backward(dout, qw, scales, K=K, group_size=gs, math="f16")
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("name", ["prefill_1b", "llama8b_gs128"])
def test_backward_f16_full_size_sampled(name):
    """Every projection at M = 512 over full-size weights, on 400 sampled
    gradient elements computed one by one by the oracle."""
    need_gpu()
    from bit_weight_only_int4_amd.workloads import make_inputs
    dev = torch.device("cuda")
    for p in CONFIGS[name]:
        if p.M != 512:
            continue
        seed = zlib.crc32(p.name.encode())
        log(f"[backward f16 full] {p.name} seed={seed}")
        _, qw, scales, _ = make_inputs(p, seed)
        g = torch.Generator().manual_seed(seed + 1)
        dout = torch.randn((p.M, p.N), generator=g)
        got, path = b.linear_backward(dout.to(dev), qw.to(dev), scales.to(dev), K=p.K,
                                      group_size=p.group_size, nibble_order=p.order,
                                      math="f16", return_path=True)
        torch.cuda.synchronize()
        assert path == "bwd_f16"
        rng = np.random.default_rng(seed)
        ms = rng.integers(0, p.M, 400)
        ks = rng.integers(0, p.K, 400)
        ref, den = orc.linear_backward_sampled(dout.numpy(), qw.numpy(), scales.numpy(), ms, ks,
                                               K=p.K, group_size=p.group_size, order=p.order)
        err = normalised_error(got.cpu().numpy()[ms, ks], ref, den)
        log(f"          max normalised error={err:.3e}")
        assert err <= BWD_TOL["bwd_f16"]


@pytest.mark.parametrize("math,M,N,K", [
    ("f16", 130, 600, 1032),   # MFMA gradient, no split over N
    ("f16", 64, 4096, 264),    # MFMA gradient, split over N (the reduce kernel's stores)
    ("f32", 3, 700, 1000),     # fp32 gradient
    ("f32", 2, 700, 1024),     # fp32 gradient, aligned rows
])
def test_backward_dx_not_16_byte_aligned(math, M, N, K):
    """d_x may start at any 4-byte boundary: a view one float into its
    buffer gets the same values and nothing outside [M, K] is written."""
    need_gpu()
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M + N + K)
    dout = torch.randn(M, N, generator=g)
    qw = torch.randint(0, 256, (N, (K + 1) // 2), dtype=torch.uint8, generator=g)
    s = 0.005 + 0.015 * torch.rand(-(-K // 32), N, generator=g)
    buf = torch.full((M + 2, K + 5), float("nan"), dtype=torch.float32, device=dev)
    dx = buf[:M, 1:K + 1]
    assert dx.data_ptr() % 16 != 0
    b.linear_backward(dout.to(dev), qw.to(dev), s.to(dev), K=K, group_size=32, math=math, dx=dx)
    torch.cuda.synchronize()
    full = buf.cpu().numpy()
    assert np.all(np.isnan(full[:, 0])) and np.all(np.isnan(full[:, K + 1:]))
    assert np.all(np.isnan(full[M:, :]))
    got = full[:M, 1:K + 1]
    ref, den = orc.linear_backward(dout.numpy(), qw.numpy(), s.numpy(), K=K, group_size=32)
    assert not np.any(np.isnan(got))
    err = normalised_error(got, ref, den)
    log(f"[case] dx unaligned {math} M={M} N={N} K={K}: max normalised error {err:.3e}")
    assert err <= (2e-3 if math == "f16" else 1e-5), err
