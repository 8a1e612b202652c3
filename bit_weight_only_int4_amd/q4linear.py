"""Python binding of the C ABI in ``include/q4linear.h`` (ctypes).

Argument marshalling only: tensors are checked, ``out`` and the workspace are
allocated with torch, and every step of the layer runs in the HIP library on
torch's current stream.  If the library is not built the first call raises;
there is no CPU fallback.
"""
import ctypes
import os
from typing import Optional

import torch

from . import build as _build

Q4_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "output overlaps an input",
          3: "workspace missing or too small", 4: "unsupported request",
          5: "HIP launch error"}
ORDERS = {"low_first": 0, "high_first": 1}
MATHS = {"auto": 0, "f32": 1, "f16": 2, "bf16": 3}  # bf16: not built (Q4_ERR_UNSUPPORTED)
PATHS = {0: "none", 1: "gemv_f32", 2: "gemm_f16", 3: "bwd_f32", 4: "bwd_f16",
         5: "gemm_f16_skinny"}
DTYPES = {torch.float32: 0, torch.float16: 1}

# exported symbols of include/q4linear.h
SYMBOLS = ("q4_linear", "q4_linear_f16_scales", "q4_linear_workspace_bytes", "q4_linear_backward",
           "q4_linear_backward_workspace_bytes", "q4_requant", "q4_unpack_codes",
           "q4_dequant", "q4_linear_noalloc", "q4_status_str", "q4_abi_version")
ABI_VERSION = 2
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _build.LIB


def lib() -> ctypes.CDLL:
    """The loaded HIP library with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is not built; run "
            "`python -c 'import __graft_entry__ as g; g.build()'` first")
    if os.path.abspath(path) == os.path.abspath(_build.TREE_LIB):
        why = _build.stale_reason(path)
        if why:
            raise RuntimeError(
                f"HIP library {path} does not match the sources: {why}; rebuild it "
                "(`python -c 'import __graft_entry__ as g; g.build()'`)")
    L = ctypes.CDLL(path)
    P, I, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.q4_linear.argtypes = [P, I, P, I, P, I, I, P, P, I, I, I, I, I32, I32, P, SZ, P, P]
    L.q4_linear.restype = I32
    L.q4_linear_f16_scales.argtypes = L.q4_linear.argtypes
    L.q4_linear_f16_scales.restype = I32
    L.q4_linear_noalloc.argtypes = [P, I, P, I, P, I, I, P, P, I, I, I, I, I32, I32, P, P]
    L.q4_linear_noalloc.restype = I32
    L.q4_linear_workspace_bytes.argtypes = [I, I, I, I, I32]
    L.q4_linear_workspace_bytes.restype = SZ
    L.q4_unpack_codes.argtypes = [P, I, I, I, I32, P, I, P]
    L.q4_unpack_codes.restype = I32
    L.q4_dequant.argtypes = [P, I, P, I, I, I, I, I32, I32, P, I, P]
    L.q4_dequant.restype = I32
    L.q4_linear_backward.argtypes = [P, I, P, I, P, I, I, P, I, I, I, I, I32, I32, P, SZ, P, P]
    L.q4_linear_backward.restype = I32
    L.q4_linear_backward_workspace_bytes.argtypes = [I, I, I, I, I32]
    L.q4_linear_backward_workspace_bytes.restype = SZ
    L.q4_requant.argtypes = [P, I, P, I, I, I, I, I32, P, I, P]
    L.q4_requant.restype = I32
    L.q4_status_str.argtypes = [I32]
    L.q4_status_str.restype = ctypes.c_char_p
    L.q4_abi_version.argtypes = []
    L.q4_abi_version.restype = I32
    _lib = L
    return L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(t: torch.Tensor, name: str, dtype) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit stride along its rows")
    return t.stride(0) if t.size(0) > 1 else max(t.size(1), t.stride(0))


def _need(ok: bool, msg: str) -> None:
    if not ok:
        raise ValueError(msg)


def _check_scales(scales: torch.Tensor, group_size: int, N: int, K: int) -> None:
    if group_size == 0:
        _need(scales.dim() == 1 and scales.numel() >= N,
              f"per-channel scales need N = {N} entries, got shape {tuple(scales.shape)}")
    elif group_size > 0:
        G = -(-K // group_size)
        _need(scales.dim() == 2 and scales.size(0) >= G and scales.size(1) >= N,
              f"grouped scales need [ceil(K / group_size), N] = [{G}, {N}], "
              f"got {tuple(scales.shape)}")


def _check_linear_extents(x: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor,
                          bias: Optional[torch.Tensor], out: Optional[torch.Tensor],
                          K: int, group_size: int) -> None:
    """Extents the C ABI does not see (it takes pitches, not sizes): an
    undersized tensor is rejected here, before anything is queued, instead
    of being read or written past its end."""
    _need(x.dim() == 2, f"x must be 2-D [M, K], got shape {tuple(x.shape)}")
    _need(x.size(1) >= K, f"x has {x.size(1)} columns, fewer than K = {K}")
    _need(qw.dim() == 2 and qw.size(1) >= (K + 1) // 2,
          f"qw needs [N, ceil(K / 2)] = [N, {(K + 1) // 2}] bytes, got {tuple(qw.shape)}")
    M, N = x.size(0), qw.size(0)
    _check_scales(scales, group_size, N, K)
    if bias is not None:
        _need(bias.dim() == 1 and bias.numel() >= N,
              f"bias needs N = {N} entries, got shape {tuple(bias.shape)}")
    if out is not None:
        _need(tuple(out.shape) == (M, N), f"out must be [M, N] = [{M}, {N}], "
                                          f"got {tuple(out.shape)}")


def workspace_bytes(M: int, N: int, K: int, group_size: int, math: str = "auto") -> int:
    return int(lib().q4_linear_workspace_bytes(M, N, K, group_size, MATHS[math]))


def linear(x: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor,
           bias: Optional[torch.Tensor] = None, *, K: Optional[int] = None,
           group_size: int, nibble_order: str = "low_first", math: str = "auto",
           out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, return_path: bool = False):
    """out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8) (+ bias[n]).

    x [M, K] float32; qw [N, ceil(K/2)] uint8; scales [ceil(K/gs), N]
    (group_size > 0) or [N] (group_size == 0), float32, or float16 for
    q4f16_1 weights (then q4_linear_f16_scales runs); bias [N] float32 or
    None.  Row strides of x, qw, scales and out are passed through as pitches.
    """
    K = x.size(1) if K is None else K
    _check_linear_extents(x, qw, scales, bias, out, K, group_size)
    ldx = _rows(x, "x", torch.float32)
    ldq = _rows(qw, "qw", torch.uint8)
    M, N = x.size(0), qw.size(0)
    if scales.dtype not in (torch.float32, torch.float16):
        raise ValueError("scales must be float32 or float16")
    entry = lib().q4_linear_f16_scales if scales.dtype == torch.float16 else lib().q4_linear
    if group_size == 0:
        if scales.dim() != 1 or scales.stride(0) != 1 or not scales.is_cuda:
            raise ValueError("per-channel scales must be a contiguous 1-D device tensor")
        lds = N
    else:
        lds = _rows(scales, "scales", scales.dtype)
    if bias is not None:
        if not bias.is_cuda or bias.dtype != torch.float32 or bias.dim() != 1 \
                or bias.stride(0) != 1:
            raise ValueError("bias must be a contiguous float32 device vector")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ldo = _rows(out, "out", torch.float32) if M > 0 and N > 0 else max(N, 1)
    need = workspace_bytes(M, N, K, group_size, math) if M > 0 and N > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    path = ctypes.c_int32(0)
    st = entry(_ptr(x), ldx, _ptr(qw), ldq, _ptr(scales), lds, group_size,
               _ptr(bias), _ptr(out), ldo, M, N, K, ORDERS[nibble_order],
               MATHS[math], _ptr(workspace), ws_bytes, _stream(),
               ctypes.byref(path))
    if st != Q4_OK:
        raise Q4Error(st, entry.__name__)
    return (out, PATHS[path.value]) if return_path else out


def linear_noalloc(x: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor,
                   bias: Optional[torch.Tensor] = None, *, out: torch.Tensor,
                   K: Optional[int] = None, group_size: int, nibble_order: str = "low_first",
                   math: str = "auto", return_path: bool = False):
    """``linear`` through q4_linear_noalloc: no device memory is allocated
    (the caller passes ``out``; the workspace is the library's own).  fp32
    scales only, as that entry point takes."""
    K = x.size(1) if K is None else K
    _check_linear_extents(x, qw, scales, bias, out, K, group_size)
    ldx = _rows(x, "x", torch.float32)
    ldq = _rows(qw, "qw", torch.uint8)
    M, N = x.size(0), qw.size(0)
    if group_size == 0:
        if scales.dim() != 1 or scales.stride(0) != 1 or not scales.is_cuda \
                or scales.dtype != torch.float32:
            raise ValueError("per-channel scales must be a contiguous float32 device vector")
        lds = N
    else:
        lds = _rows(scales, "scales", torch.float32)
    if bias is not None:
        if not bias.is_cuda or bias.dtype != torch.float32 or bias.dim() != 1 \
                or bias.stride(0) != 1:
            raise ValueError("bias must be a contiguous float32 device vector")
    ldo = _rows(out, "out", torch.float32) if M > 0 and N > 0 else max(N, 1)
    path = ctypes.c_int32(0)
    st = lib().q4_linear_noalloc(_ptr(x), ldx, _ptr(qw), ldq, _ptr(scales), lds, group_size,
                                 _ptr(bias), _ptr(out), ldo, M, N, K, ORDERS[nibble_order],
                                 MATHS[math], _stream(), ctypes.byref(path))
    if st != Q4_OK:
        raise Q4Error(st, "q4_linear_noalloc")
    return (out, PATHS[path.value]) if return_path else out


def _scales_pitch(scales: torch.Tensor, group_size: int, N: int) -> int:
    if group_size == 0:
        if scales.dim() != 1 or scales.stride(0) != 1 or not scales.is_cuda:
            raise ValueError("per-channel scales must be a contiguous 1-D device tensor")
        if scales.dtype != torch.float32:
            raise ValueError("scales must be float32")
        return N
    return _rows(scales, "scales", torch.float32)


def backward_workspace_bytes(M: int, N: int, K: int, group_size: int,
                             math: str = "auto") -> int:
    return int(lib().q4_linear_backward_workspace_bytes(M, N, K, group_size, MATHS[math]))


def linear_backward(dout: torch.Tensor, qw: torch.Tensor, scales: torch.Tensor, *, K: int,
                    group_size: int, nibble_order: str = "low_first", math: str = "auto",
                    dx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, return_path: bool = False):
    """dx[m, k] = sum_n dout[m, n] * (q[n, k] - 8) * s[g(k), n]: the input
    gradient of ``linear``.  dout [M, N] float32; qw and scales as in linear."""
    _need(dout.dim() == 2 and qw.dim() == 2 and qw.size(1) >= (K + 1) // 2,
          f"dout must be 2-D and qw [N, ceil(K / 2)] = [N, {(K + 1) // 2}] bytes, "
          f"got {tuple(dout.shape)} and {tuple(qw.shape)}")
    _check_scales(scales, group_size, qw.size(0), K)
    if dx is not None:
        _need(tuple(dx.shape) == (dout.size(0), K),
              f"dx must be [M, K] = [{dout.size(0)}, {K}], got {tuple(dx.shape)}")
    lddo = _rows(dout, "dout", torch.float32)
    ldq = _rows(qw, "qw", torch.uint8)
    M, N = dout.size(0), qw.size(0)
    if dout.size(1) != N:
        raise ValueError("dout must have one column per weight row")
    lds = _scales_pitch(scales, group_size, N)
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=dout.device)
    lddx = _rows(dx, "dx", torch.float32) if M > 0 else K
    need = backward_workspace_bytes(M, N, K, group_size, math) if M > 0 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dout.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    path = ctypes.c_int32(0)
    st = lib().q4_linear_backward(_ptr(dout), lddo, _ptr(qw), ldq, _ptr(scales), lds,
                                  group_size, _ptr(dx), lddx, M, N, K, ORDERS[nibble_order],
                                  MATHS[math], _ptr(workspace), ws_bytes, _stream(),
                                  ctypes.byref(path))
    if st != Q4_OK:
        raise Q4Error(st, "q4_linear_backward")
    return (dx, PATHS[path.value]) if return_path else dx


def requant(latent: torch.Tensor, scales: torch.Tensor, *, group_size: int,
            nibble_order: str = "low_first", qw: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed codes [N, ceil(K/2)] uint8 of fp32 latent weights [N, K]:
    clamp(round(latent / s), -8, 7) + 8, zero scale -> 8."""
    _need(latent.dim() == 2, f"latent must be 2-D [N, K], got {tuple(latent.shape)}")
    N, K = latent.shape
    _check_scales(scales, group_size, N, K)
    if qw is not None:
        _need(qw.dim() == 2 and qw.size(0) == N and qw.size(1) >= (K + 1) // 2,
              f"qw must be [N, >= ceil(K / 2)] = [{N}, >= {(K + 1) // 2}], got {tuple(qw.shape)}")
    ldl = _rows(latent, "latent", torch.float32)
    lds = _scales_pitch(scales, group_size, N)
    if qw is None:
        qw = torch.empty((N, (K + 1) // 2), dtype=torch.uint8, device=latent.device)
    ldq = _rows(qw, "qw", torch.uint8)
    st = lib().q4_requant(_ptr(latent), ldl, _ptr(scales), lds, group_size, N, K,
                          ORDERS[nibble_order], _ptr(qw), ldq, _stream())
    if st != Q4_OK:
        raise Q4Error(st, "q4_requant")
    return qw


def unpack_codes(qw: torch.Tensor, K: int, nibble_order: str = "low_first") -> torch.Tensor:
    """Signed codes q - 8 as int8 [N, K]."""
    _need(qw.dim() == 2 and qw.size(1) >= (K + 1) // 2,
          f"qw needs [N, ceil(K / 2)] = [N, {(K + 1) // 2}] bytes, got {tuple(qw.shape)}")
    ldq = _rows(qw, "qw", torch.uint8)
    N = qw.size(0)
    codes = torch.empty((N, K), dtype=torch.int8, device=qw.device)
    st = lib().q4_unpack_codes(_ptr(qw), ldq, N, K, ORDERS[nibble_order], _ptr(codes), K,
                               _stream())
    if st != Q4_OK:
        raise Q4Error(st, "q4_unpack_codes")
    return codes


def dequant(qw: torch.Tensor, scales: torch.Tensor, K: int, group_size: int,
            nibble_order: str = "low_first", dtype=torch.float32) -> torch.Tensor:
    """Dequantized weight [N, K]: float32 RN32((q-8)*s) or float16 RN16((q-8)*RN16(s))."""
    _need(qw.dim() == 2 and qw.size(1) >= (K + 1) // 2,
          f"qw needs [N, ceil(K / 2)] = [N, {(K + 1) // 2}] bytes, got {tuple(qw.shape)}")
    _check_scales(scales, group_size, qw.size(0), K)
    ldq = _rows(qw, "qw", torch.uint8)
    N = qw.size(0)
    lds = N if group_size == 0 else _rows(scales, "scales", torch.float32)
    w = torch.empty((N, K), dtype=dtype, device=qw.device)
    st = lib().q4_dequant(_ptr(qw), ldq, _ptr(scales), lds, group_size, N, K,
                          ORDERS[nibble_order], DTYPES[dtype], _ptr(w), K, _stream())
    if st != Q4_OK:
        raise Q4Error(st, "q4_dequant")
    return w
