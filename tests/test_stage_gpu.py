"""GPU bit-exactness of the unpack and dequant stages against the oracle.

The exported stages run the same device functions the layer's kernels use;
the bar is bit-identical output.
"""
import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs
from oracle import q4_oracle as orc
from tests.gpu_util import log, need_gpu

pytestmark = pytest.mark.gpu


def _check(qw, scales, K, gs, order):
    log(f"[stage] N={qw.shape[0]} K={K} gs={gs} order={order}")
    dev = torch.device("cuda")
    qd, sd = qw.to(dev), scales.to(dev)
    codes = b.unpack_codes(qd, K, order).cpu().numpy()
    assert np.array_equal(codes, orc.unpack_codes(qw.numpy(), K, order))
    w32 = b.dequant(qd, sd, K, gs, order, torch.float32).cpu().numpy()
    ref32 = orc.dequant_f32(qw.numpy(), scales.numpy(), K, gs, order)
    assert np.array_equal(w32.view(np.uint32), ref32.view(np.uint32))
    w16 = b.dequant(qd, sd, K, gs, order, torch.float16).cpu()
    got16 = w16.view(torch.int16).numpy().view(np.uint16)
    ref16 = orc.dequant_f16_bits(qw.numpy(), scales.numpy(), K, gs, order)
    # IEEE 754 leaves the sign and payload of a default NaN open (0 * inf
    # when a scale overflows binary16): NaN must meet NaN, every other value
    # must match bit for bit
    nan_got = (got16 & 0x7C00) == 0x7C00
    nan_got &= (got16 & 0x03FF) != 0
    nan_ref = ((ref16 & 0x7C00) == 0x7C00) & ((ref16 & 0x03FF) != 0)
    assert np.array_equal(nan_got, nan_ref)
    assert np.array_equal(got16[~nan_got], ref16[~nan_ref])


@pytest.mark.parametrize("K,N,gs", [(256, 128, 32), (2008, 33, 0), (2007, 40, 32),
                                    (1000, 17, 8), (130, 9, 100), (7, 3, 3), (1, 5, 0)])
@pytest.mark.parametrize("order", ["low_first", "high_first"])
def test_stages_bit_exact(K, N, gs, order):
    need_gpu()
    g = torch.Generator().manual_seed(K * 31 + N)
    qw = torch.randint(0, 256, (N, (K + 1) // 2), generator=g, dtype=torch.uint8)
    shape = (N,) if gs == 0 else ((K + gs - 1) // gs, N)
    scales = torch.rand(shape, generator=g) * 0.02 + 0.001
    _check(qw, scales, K, gs, order)


def test_dequant_f16_wide_scale_range():
    """Scales from 1e-9 to 1e5: binary16 subnormals, underflow to zero and
    overflow to infinity all round as the oracle's IEEE definition says."""
    need_gpu()
    g = torch.Generator().manual_seed(77)
    N, K, gs = 64, 512, 32
    qw = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    mant = torch.rand((K // gs, N), generator=g) + 0.5
    expo = torch.randint(-9, 6, (K // gs, N), generator=g).to(torch.float32)
    scales = (mant * torch.pow(10.0, expo)).to(torch.float32)
    _check(qw, scales, K, gs, "low_first")


@pytest.mark.parametrize("name", list(CONFIGS))
def test_stages_on_every_workload(name):
    """Each workload's weights (a sample of rows for the large ones)."""
    need_gpu()
    seen = set()
    for p in CONFIGS[name]:
        key = (p.K, p.N, p.group_size, p.order)
        if key in seen:
            continue
        seen.add(key)
        _, qw, scales, _ = make_inputs(p.with_m(1), 0)
        rows = torch.arange(qw.shape[0])
        if qw.shape[0] > 512:
            rows = torch.randperm(qw.shape[0], generator=torch.Generator().manual_seed(1))[:512]
            rows, _ = rows.sort()
        q_s = qw[rows].contiguous()
        s_s = scales[rows].contiguous() if p.group_size == 0 else scales[:, rows].contiguous()
        _check(q_s, s_s, p.K, p.group_size, p.order)
