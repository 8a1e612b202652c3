"""ctypes front end of the fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the GPU path; it takes plain
numpy arrays and returns numpy arrays.

Array conventions (all C-contiguous, row pitch = the array's second dim):
  x       float32 [M, ldx]      activations, ldx >= K
  qw      uint8   [N, ldq]      packed nibbles, ldq >= ceil(K / 2)
  scales  float32 [G, lds]      grouped (G = ceil(K / group_size), lds >= N)
          float32 [N]           per-channel (group_size == 0)
  bias    float32 [N] or None
  order   "low_first"  (even k in the low nibble; q4gsw packer)
          "high_first" (even k in the high nibble; qcs4w packer)
The nibble order and scale indexing follow page 5, "[ExecuTorch][WebGPU] Add
linear_qcs4w op", Constraints (2) and Solution; the signed offset follows
page 3, "Add fp32 matmul ops (mm, bmm, linear)", stack entry #20943.

Pages cited by number (the texts this layer is written from):
  page 1: ExecuTorch PR #20815, "[WebGPU] Add 256-thread steel q4gsw prefill GEMM"
          (its stack entries #20730 ... #20801);
  page 2: ExecuTorch PR #20847, "[WebGPU] Add optimized linear_fp32 op";
  page 3: ExecuTorch PR #21070, "Add fp32 matmul ops (mm, bmm, linear)"
          (its stack entries #20917 ... #21005);
  page 4: Apache TVM PR #20425, the dlight GEMV rule's webgpu branch;
  page 5: ExecuTorch PR #21211, "[WebGPU] Add linear_qcs4w op".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_ORDERS = {"low_first": 0, "high_first": 1}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        if os.path.abspath(_build.LIB) == os.path.abspath(_build.TREE_LIB):
            why = _build.stale_reason(_build.LIB)
            if why:
                raise RuntimeError(f"oracle library {_build.LIB} does not match q4_oracle.c: "
                                   f"{why}; rebuild it (oracle.build.build())")
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        C = ctypes.c_int
        lib.q4o_rn_f16_bits.argtypes = [ctypes.c_double]
        lib.q4o_rn_f16_bits.restype = ctypes.c_uint16
        lib.q4o_f16_value.argtypes = [ctypes.c_uint16]
        lib.q4o_f16_value.restype = ctypes.c_double
        lib.q4o_round_f16.argtypes = [P, I, P]
        lib.q4o_f16_values.argtypes = [P, I, P]
        lib.q4o_unpack_codes.argtypes = [P, I, I, I, C, P, I]
        lib.q4o_dequant_f64.argtypes = [P, I, P, I, I, I, I, C, P, I]
        lib.q4o_dequant_f32.argtypes = [P, I, P, I, I, I, I, C, P, I]
        lib.q4o_dequant_f16.argtypes = [P, I, P, I, I, I, I, C, P, I]
        lib.q4o_linear.argtypes = [P, I, P, I, P, I, I, P, I, I, I, C, P, P]
        lib.q4o_linear_sampled.argtypes = [P, I, P, I, P, I, I, P, I, C, I,
                                           P, P, P, P]
        lib.q4o_linear_backward.argtypes = [P, I, P, I, P, I, I, I, I, I, C,
                                            P, P]
        lib.q4o_linear_backward_sampled.argtypes = [P, I, P, I, P, I, I, I, C,
                                                    I, P, P, P, P]
        lib.q4o_requant.argtypes = [P, I, P, I, I, I, I, C, P, I]
        lib.q4o_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _order(order):
    if order not in _ORDERS:
        raise ValueError(f"unknown nibble order {order!r}")
    return _ORDERS[order]


def _check_c(a, dtype, ndim, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or a.ndim != ndim \
            or not a.flags.c_contiguous:
        raise ValueError(f"{name}: need a C-contiguous {dtype} array of "
                         f"rank {ndim}")


def _weights(qw, scales, group_size, K):
    _check_c(qw, np.uint8, 2, "qw")
    N, ldq = qw.shape
    if ldq < (K + 1) // 2:
        raise ValueError("qw row pitch below ceil(K/2)")
    if group_size == 0:
        _check_c(scales, np.float32, 1, "scales")
        if scales.shape[0] < N:
            raise ValueError("per-channel scales shorter than N")
        lds = 0
    else:
        _check_c(scales, np.float32, 2, "scales")
        G = -(-K // group_size)
        if scales.shape[0] < G or scales.shape[1] < N:
            raise ValueError("grouped scales smaller than [ceil(K/gs), N]")
        lds = scales.shape[1]
    return N, ldq, lds


def max_threads() -> int:
    return int(_load().q4o_max_threads())


def rn_f16_bits(values) -> np.ndarray:
    """Binary16 bit patterns of float32 values, rounded to nearest even."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().q4o_round_f16(_ptr(v), v.size, _ptr(out))
    return out


def f16_value(bits: int) -> float:
    return float(_load().q4o_f16_value(int(bits)))


def f16_scales_to_f32(bits) -> np.ndarray:
    """Binary16 scales (uint16 bit patterns) as their exact float32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _load().q4o_f16_values(_ptr(b), b.size, _ptr(out))
    return out


def linear_f16_scales(x, qw, scale_bits, bias=None, *, K, group_size, order="low_first"):
    """The layer with binary16 scales (q4f16_1 format): the scales widened
    exactly, then linear()."""
    return linear(x, qw, f16_scales_to_f32(scale_bits), bias, K=K, group_size=group_size,
                  order=order)


def unpack_codes(qw, K, order="low_first") -> np.ndarray:
    """Signed codes c = q - 8 as int8 [N, K]."""
    _check_c(qw, np.uint8, 2, "qw")
    N, ldq = qw.shape
    codes = np.empty((N, K), dtype=np.int8)
    _load().q4o_unpack_codes(_ptr(qw), ldq, N, K, _order(order), _ptr(codes), K)
    return codes


def dequant_f64(qw, scales, K, group_size, order="low_first") -> np.ndarray:
    N, ldq, lds = _weights(qw, scales, group_size, K)
    w = np.empty((N, K), dtype=np.float64)
    _load().q4o_dequant_f64(_ptr(qw), ldq, _ptr(scales), lds, group_size, N, K,
                            _order(order), _ptr(w), K)
    return w


def dequant_f32(qw, scales, K, group_size, order="low_first") -> np.ndarray:
    N, ldq, lds = _weights(qw, scales, group_size, K)
    w = np.empty((N, K), dtype=np.float32)
    _load().q4o_dequant_f32(_ptr(qw), ldq, _ptr(scales), lds, group_size, N, K,
                            _order(order), _ptr(w), K)
    return w


def dequant_f16_bits(qw, scales, K, group_size, order="low_first") -> np.ndarray:
    N, ldq, lds = _weights(qw, scales, group_size, K)
    w = np.empty((N, K), dtype=np.uint16)
    _load().q4o_dequant_f16(_ptr(qw), ldq, _ptr(scales), lds, group_size, N, K,
                            _order(order), _ptr(w), K)
    return w


def linear(x, qw, scales, bias=None, *, K, group_size, order="low_first"):
    """fp64 result and normaliser: (out [M, N], den [M, N]), both float64.

    den[m, n] = sum_k |x[m, k] * w[n, k]|.
    """
    _check_c(x, np.float32, 2, "x")
    M, ldx = x.shape
    if ldx < K:
        raise ValueError("x row pitch below K")
    N, ldq, lds = _weights(qw, scales, group_size, K)
    if bias is not None:
        _check_c(bias, np.float32, 1, "bias")
        if bias.shape[0] < N:
            raise ValueError("bias shorter than N")
    out = np.empty((M, N), dtype=np.float64)
    den = np.empty((M, N), dtype=np.float64)
    _load().q4o_linear(_ptr(x), ldx, _ptr(qw), ldq, _ptr(scales), lds,
                       group_size, _ptr(bias), M, N, K, _order(order),
                       _ptr(out), _ptr(den))
    return out, den


def linear_sampled(x, qw, scales, bias, ms, ns, *, K, group_size,
                   order="low_first"):
    """fp64 results at the output coordinates (ms[i], ns[i])."""
    _check_c(x, np.float32, 2, "x")
    M, ldx = x.shape
    N, ldq, lds = _weights(qw, scales, group_size, K)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be equal-length vectors")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0
                    or ns.max() >= N):
        raise ValueError("sample coordinate out of range")
    if bias is not None:
        _check_c(bias, np.float32, 1, "bias")
    out = np.empty(ms.shape, dtype=np.float64)
    den = np.empty(ms.shape, dtype=np.float64)
    _load().q4o_linear_sampled(_ptr(x), ldx, _ptr(qw), ldq, _ptr(scales), lds,
                               group_size, _ptr(bias), K, _order(order),
                               ms.size, _ptr(ms), _ptr(ns), _ptr(out),
                               _ptr(den))
    return out, den


def linear_backward(dout, qw, scales, *, K, group_size, order="low_first"):
    """fp64 input gradient and normaliser: (dx [M, K], den [M, K]).

    dx[m, k] = sum_n dout[m, n] * w[n, k]; den = sum_n |dout[m, n] * w[n, k]|
    (page 3, stack entry #20943).
    """
    _check_c(dout, np.float32, 2, "dout")
    N, ldq, lds = _weights(qw, scales, group_size, K)
    M, lddo = dout.shape
    if lddo < N:
        raise ValueError("dout row pitch below N")
    dx = np.empty((M, K), dtype=np.float64)
    den = np.empty((M, K), dtype=np.float64)
    _load().q4o_linear_backward(_ptr(dout), lddo, _ptr(qw), ldq, _ptr(scales), lds,
                                group_size, M, N, K, _order(order), _ptr(dx), _ptr(den))
    return dx, den


def linear_backward_sampled(dout, qw, scales, ms, ks, *, K, group_size,
                            order="low_first"):
    """fp64 input-gradient elements at (ms[i], ks[i])."""
    _check_c(dout, np.float32, 2, "dout")
    N, ldq, lds = _weights(qw, scales, group_size, K)
    M, lddo = dout.shape
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    if ms.shape != ks.shape or ms.ndim != 1:
        raise ValueError("ms and ks must be equal-length vectors")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ks.min() < 0
                    or ks.max() >= K):
        raise ValueError("sample coordinate out of range")
    out = np.empty(ms.shape, dtype=np.float64)
    den = np.empty(ms.shape, dtype=np.float64)
    _load().q4o_linear_backward_sampled(_ptr(dout), lddo, _ptr(qw), ldq, _ptr(scales),
                                        lds, group_size, N, _order(order), ms.size,
                                        _ptr(ms), _ptr(ks), _ptr(out), _ptr(den))
    return out, den


def requant(latent, scales, *, group_size, order="low_first", ldq=None, fill=0):
    """Packed codes uint8 [N, ldq] of fp32 latent weights [N, K]:
    clamp(round(latent / s), -8, 7) + 8 with the quotient in fp32 and ties to
    even, zero scale -> code 8, odd K padded with code 8 (page 3, stack
    entries #20945, #20946).  Bytes past ceil(K/2) hold `fill`."""
    _check_c(latent, np.float32, 2, "latent")
    N, K = latent.shape
    Kp = (K + 1) // 2
    ldq = Kp if ldq is None else ldq
    if ldq < Kp:
        raise ValueError("ldq below ceil(K/2)")
    qw = np.full((N, ldq), fill, dtype=np.uint8)
    _, _, lds = _weights(qw, scales, group_size, K)
    _load().q4o_requant(_ptr(latent), K, _ptr(scales), lds, group_size, N, K,
                        _order(order), _ptr(qw), ldq)
    return qw
