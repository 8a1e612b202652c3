"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole output is computed on the GPU and every element
is checked against the oracle (fp64, computed on the host's cores), at the
bar of the path that ran, with NaN-free and guard checks over the whole
output buffer.
"""
import time

import numpy as np
import pytest

from bit_weight_only_int4_amd.workloads import CONFIGS, make_inputs
from tests.gpu_util import TOL, log, need_gpu, normalised_error, oracle_full, run_gpu

pytestmark = pytest.mark.gpu

CASES = [(name, i) for name in CONFIGS for i in range(len(CONFIGS[name]))]


@pytest.mark.parametrize("name,i", CASES, ids=[f"{n}-{i}" for n, i in CASES])
def test_full_size_every_element(name, i):
    need_gpu()
    p = CONFIGS[name][i]
    log(f"[full] {p.name} M={p.M} K={p.K} N={p.N} gs={p.group_size} order={p.order}")
    x, qw, s, bias = make_inputs(p, 0)
    out, path, guards = run_gpu(x, qw, s, bias, K=p.K, gs=p.group_size, order=p.order)
    assert guards, "write outside [M, N]"
    assert not np.isnan(out).any()
    t0 = time.time()
    ref, den = oracle_full(x, qw, s, bias, K=p.K, gs=p.group_size, order=p.order)
    err = normalised_error(out, ref, den)
    log(f"       path={path} elements={out.size} max normalised error={err:.3e} "
        f"(tol {TOL[path]:.0e}; oracle {time.time() - t0:.1f} s)")
    assert err <= TOL[path]
