"""Shared helpers of the GPU parity tests: run the HIP path through the
binding and compare it with the fp64 oracle on the same seeded inputs.

Bar (normalised by den = sum_k |x * w|, computed by the oracle):
  * pure-fp32 GEMV path:           max |gpu - ref| / den <= 1e-5
  * binary16-operand MFMA path:    max |gpu - ref| / den <= 2e-3
  * where den == 0 the output must equal the oracle exactly (it is the bias
    or zero).
"""
import numpy as np
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b
from oracle import q4_oracle as orc

TOL = {"gemv_f32": 1e-5, "gemm_f16": 2e-3, "gemm_f16_skinny": 2e-3}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(msg):
    print(msg, flush=True)


def normalised_error(gpu: np.ndarray, ref: np.ndarray, den: np.ndarray):
    gpu = gpu.astype(np.float64)
    diff = np.abs(gpu - ref)
    zero = den == 0
    if np.any(zero):
        assert np.array_equal(gpu[zero], ref[zero]), "den == 0 outputs must be exact"
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, den))
    return float(rel.max()) if rel.size else 0.0


def run_gpu(x, qw, scales, bias, *, K, gs, order, math="auto", pad=(0, 0, 0, 0),
            poison=True):
    """Run the HIP path on padded device copies.  pad = extra elements on the
    row pitch of (x, qw, scales, out).  The output buffer is NaN-poisoned and
    has 2 guard rows and pad[3] guard columns; returns (out [M, N] numpy,
    path, guards_intact)."""
    dev = torch.device("cuda")
    M, N = x.shape[0], qw.shape[0]

    def padded(t, extra, fill):
        if t.dim() == 1 or extra == 0:
            return t.to(dev).contiguous()
        buf = torch.full((t.shape[0], t.shape[1] + extra), fill, dtype=t.dtype, device=dev)
        buf[:, : t.shape[1]] = t.to(dev)
        return buf[:, : t.shape[1]]

    xd = padded(x, pad[0], float("nan"))
    qd = padded(qw, pad[1], 0xFF)
    sd = padded(scales, pad[2], float("nan"))
    bd = None if bias is None else bias.to(dev).contiguous()
    ldo = N + pad[3]
    obuf = torch.full((M + 2, max(ldo, 1)), float("nan") if poison else 0.0,
                      dtype=torch.float32, device=dev)
    out = obuf[:M, :N]
    res, path = b.linear(xd, qd, sd, bd, K=K, group_size=gs, nibble_order=order, math=math,
                         out=out, return_path=True)
    torch.cuda.synchronize()
    full = obuf.cpu().numpy()
    guards = bool(np.all(np.isnan(full[M:, :])) and np.all(np.isnan(full[:M, N:])))
    return full[:M, :N].copy(), path, guards


def oracle_full(x, qw, scales, bias, *, K, gs, order):
    return orc.linear(x.numpy(), qw.numpy(), scales.numpy(),
                      None if bias is None else bias.numpy(), K=K, group_size=gs,
                      order=order)


def check_case(x, qw, scales, bias, *, K, gs, order, math="auto", pad=(0, 0, 0, 0),
               label=""):
    log(f"[case] {label} M={x.shape[0]} K={K} N={qw.shape[0]} gs={gs} order={order} "
        f"math={math} pad={pad}")
    out, path, guards = run_gpu(x, qw, scales, bias, K=K, gs=gs, order=order, math=math,
                                pad=pad)
    ref, den = oracle_full(x, qw, scales, bias, K=K, gs=gs, order=order)
    assert guards, "write outside [M, N] (NaN guard slots overwritten)"
    assert not np.any(np.isnan(out)), "NaN in the output"
    err = normalised_error(out, ref, den)
    log(f"       path={path} max normalised error={err:.3e} (tol {TOL[path]:.0e})")
    assert err <= TOL[path], (path, err)
    return out, path, err
