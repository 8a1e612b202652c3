"""GPU parity where the weight matrix is larger than 4 GiB: byte offsets of
the rows past 2^21 exceed 2^32, so every kernel that addresses the weights
through 32-bit buffer offsets (the streaming GEMV, the few-row kernel, the
pipelined GEMM) must be set aside for the kernels that address them with
64-bit pointers, and those must reach the rows past 4 GiB.

Row n of the weights is a fixed function of n (row n % 4099 of a seeded
random block, XORed with a byte hashed from n), and a grouped scale is an
exact binary fraction hashed from (g, n): the device builds the 4 GiB array
itself, and the oracle gets only the sampled rows, built the same way on the
host.  Outputs are sampled (the rows at the end of the array, the rows
around the 2^32-byte boundary, random rows) and checked against the fp64
oracle at the path's bar.
"""
import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from oracle import q4_oracle as orc
from tests.gpu_util import TOL, log, need_gpu

pytestmark = pytest.mark.gpu

K = 4096
KP = K // 2
N = (1 << 21) + 5  # N * KP = 2^32 + 10240 bytes: rows >= 2^21 start past 4 GiB
BASE_ROWS = 4099


def base_block():
    rng = np.random.default_rng(77)
    return rng.integers(0, 256, size=(BASE_ROWS, KP), dtype=np.uint8)


def row_key(n):
    """one byte per row index (numpy or torch int64 in, same dtype out)"""
    return ((n * 2654435761) >> 13) & 0xFF


def host_rows(base, ns):
    keys = row_key(ns.astype(np.int64)).astype(np.uint8)
    return np.bitwise_xor(base[ns % BASE_ROWS], keys[:, None])


def scale_value(g, n):
    """an exact binary fraction in [500, 1500) / 2^16"""
    return ((g * 7919 + n * 104729) % 1000 + 500) / 65536.0


def bias_value(n):
    """an exact binary fraction in [-1000, 1000) / 2^16"""
    return ((n * 48271) % 2000 - 1000) / 65536.0


@pytest.fixture(scope="module")
def big():
    need_gpu()
    free, _ = torch.cuda.mem_get_info()
    if free < 12 * (1 << 30):
        pytest.skip("needs about 12 GiB of free device memory")
    dev = torch.device("cuda")
    base = base_block()
    reps = -(-N // BASE_ROWS)
    qd = torch.from_numpy(base).to(dev).repeat(reps, 1)[:N]
    keys = row_key(torch.arange(N, dtype=torch.int64, device=dev)).to(torch.uint8)
    qd.bitwise_xor_(keys[:, None])
    torch.cuda.synchronize()
    assert qd.is_contiguous() and qd.shape == (N, KP)
    return base, qd


@pytest.mark.parametrize("M,gs,math,expect", [
    (1, 0, "auto", "gemv_f32"),      # one-pass GEMV (the streaming one needs offsets < 2^32)
    (1, 128, "auto", "gemv_f32"),
    (2, 0, "f32", "gemv_f32"),       # low-batch GEMV
    (4, 128, "auto", "gemm_f16"),    # general tiled GEMM (few-row and pipelined need < 2^32)
    (64, 0, "auto", "gemm_f16"),
])
def test_weights_past_4_gib(big, M, gs, math, expect):
    base, qd = big
    dev = torch.device("cuda")
    rng = np.random.default_rng(M * 7 + gs)
    x = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
    G = 1 if gs == 0 else K // gs
    n_all = torch.arange(N, dtype=torch.int64, device=dev)
    g_all = torch.arange(G, dtype=torch.int64, device=dev)[:, None]
    sd = scale_value(g_all, n_all[None, :]).to(torch.float32)
    if gs == 0:
        sd = sd[0].contiguous()
    bd = bias_value(n_all).to(torch.float32)
    out, path = b.linear(torch.from_numpy(x).to(dev), qd, sd, bd, K=K, group_size=gs,
                         math=math, return_path=True)
    torch.cuda.synchronize()
    log(f"[large] M={M} K={K} N={N} gs={gs} path={path}")
    assert path == expect
    ns = np.concatenate([np.arange(N - 40, N), np.arange((1 << 21) - 24, (1 << 21) + 5),
                         rng.integers(0, N, size=40), np.arange(0, 8)]).astype(np.int64)
    ms = rng.integers(0, M, size=ns.size).astype(np.int64)
    ms[:2] = [0, M - 1]
    got = out[torch.from_numpy(ms).to(dev), torch.from_numpy(ns).to(dev)].cpu().numpy()
    # the oracle on the sampled rows alone: row i of the compact arrays is row ns[i]
    qh = host_rows(base, ns)
    gh = np.arange(G, dtype=np.int64)[:, None]
    sh = scale_value(gh, ns[None, :]).astype(np.float32)
    if gs == 0:
        sh = np.ascontiguousarray(sh[0])
    bh = bias_value(ns).astype(np.float32)
    assert np.array_equal(qd[torch.from_numpy(ns).to(dev)].cpu().numpy(), qh)
    idx = np.arange(ns.size, dtype=np.int64)
    ref, den = orc.linear_sampled(x, qh, sh, bh, ms, idx, K=K, group_size=gs, order="low_first")
    err = np.abs(got.astype(np.float64) - ref) / den
    log(f"        sampled {ns.size} outputs, max normalised error {err.max():.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL[path]
