"""q4_linear_noalloc (the entry point for callers that cannot allocate)
against q4_linear on the GPU, through the C ABI.

Both run the same kernels with the same plan, so the outputs must be
bit-identical; each is also held to the oracle's tolerance.  Calls come in
pairs, the second on a smaller input than the first, so the second reuses a
scratch array that holds the first call's data: nothing in it may leak into
the result.
"""
import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import make_inputs, small_projection
from tests.gpu_util import TOL, log, need_gpu, normalised_error, oracle_full

pytestmark = pytest.mark.gpu

# (M, K, N, group_size, order): shapes whose plans use the workspace
# (binary16 activations, split-K partials, a split low-batch GEMV) and one
# that needs none
PAIRS = [
    ((64, 8192, 2048, 32, "low_first"), (17, 2048, 640, 32, "low_first")),
    ((512, 2048, 2048, 128, "high_first"), (96, 1024, 384, 0, "high_first")),
    ((1, 20480, 512, 32, "low_first"), (1, 18432, 200, 64, "low_first")),
    ((4, 8192, 1024, 32, "low_first"), (3, 8192, 130, 0, "high_first")),
    ((1, 2048, 1024, 32, "low_first"), (1, 2048, 96, 0, "high_first")),
    # few-row kernel over three row blocks with K split for LDS, then K % 32 != 0
    ((90, 8192, 2048, 32, "low_first"), (65, 2008, 3000, 0, "high_first")),
]


def _run(shape, seed):
    M, K, N, gs, order = shape
    p = small_projection(M, K, N, gs, order=order, has_bias=(seed % 2 == 0))
    x, qw, s, bias = make_inputs(p, seed)
    dev = torch.device("cuda")
    xd, qd, sd = x.to(dev), qw.to(dev), s.to(dev)
    bd = None if bias is None else bias.to(dev)
    need = b.workspace_bytes(M, N, K, gs)
    assert need <= b.NOALLOC_SCRATCH_BYTES
    log(f"[noalloc] M={M} K={K} N={N} gs={gs} order={order} workspace={need} B")
    ref_out, ref_path = b.linear(xd, qd, sd, bd, K=K, group_size=gs, nibble_order=order,
                                 return_path=True)
    out = torch.full((M, N), float("nan"), device=dev)
    got, path = b.linear_noalloc(xd, qd, sd, bd, out=out, K=K, group_size=gs,
                                 nibble_order=order, return_path=True)
    torch.cuda.synchronize()
    assert path == ref_path
    g, r = got.cpu().numpy(), ref_out.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), "differs from q4_linear"
    ref, den = oracle_full(x, qw, s, bias, K=K, gs=gs, order=order)
    err = normalised_error(g, ref, den)
    log(f"       path={path} bit-identical to q4_linear, max normalised error {err:.3e}")
    assert err <= TOL[path]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"pair{i}" for i in range(len(PAIRS))])
def test_noalloc_matches_linear_on_consecutive_calls(first, second):
    need_gpu()
    _run(first, 1)
    _run(second, 2)


def test_noalloc_rejects_a_workspace_beyond_its_array():
    need_gpu()
    # 2048 x 32768 activations in binary16 alone are 128 MiB
    M, K, N = 2048, 32768, 256
    assert b.workspace_bytes(M, N, K, 32) > b.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    x = torch.zeros((M, K), device=dev)
    qw = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    s = torch.zeros((K // 32, N), device=dev)
    out = torch.full((M, N), float("nan"), device=dev)
    with pytest.raises(b.Q4Error) as e:
        b.linear_noalloc(x, qw, s, None, out=out, K=K, group_size=32)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "nothing may be written on error"
