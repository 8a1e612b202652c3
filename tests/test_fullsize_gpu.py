"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole output is computed on the GPU and a seeded sample
of outputs is checked against the oracle one by one (plus NaN-free and
guard checks over the whole output).
"""
import zlib

import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs
from oracle import q4_oracle as orc
from tests.gpu_util import TOL, log, need_gpu, run_gpu

pytestmark = pytest.mark.gpu

CASES = [(name, i) for name in CONFIGS for i in range(len(CONFIGS[name]))]


@pytest.mark.parametrize("name,i", CASES, ids=[f"{n}-{i}" for n, i in CASES])
def test_full_size_sampled(name, i):
    need_gpu()
    p = CONFIGS[name][i]
    log(f"[full] {p.name}")
    x, qw, s, bias = make_inputs(p, 0)
    out, path, guards = run_gpu(x, qw, s, bias, K=p.K, gs=p.group_size, order=p.order)
    assert guards, "write outside [M, N]"
    assert not np.isnan(out).any()
    rng = np.random.default_rng(zlib.crc32(p.name.encode()))
    P = 400
    ms = rng.integers(0, p.M, P)
    ns = rng.integers(0, p.N, P)
    # always include the last row / column (ragged tails)
    ms[:4] = [p.M - 1, p.M - 1, 0, p.M - 1]
    ns[:4] = [p.N - 1, 0, p.N - 1, p.N // 2]
    ref, den = orc.linear_sampled(x.numpy(), qw.numpy(), s.numpy(),
                                  None if bias is None else bias.numpy(), ms, ns, K=p.K,
                                  group_size=p.group_size, order=p.order)
    err = np.abs(out[ms, ns].astype(np.float64) - ref) / den
    log(f"       path={path} max normalised error={err.max():.3e}")
    assert err.max() <= TOL[path]
