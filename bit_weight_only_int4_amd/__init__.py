"""Weight-only 4-bit linear layer for AMD MI355X (gfx950).

    out[m, n] = sum_k x[m, k] * s[g(k), n] * (q[n, k] - 8)  (+ bias[n])

The layer runs in hand-written HIP kernels behind the C ABI of
``include/q4linear.h``: an fp32 streaming GEMV for M == 1 (decode) and a
binary16 MFMA GEMM with fp32 accumulation for M > 1 (prefill), plus the
input gradient and re-quantization of the weights for training.  This package
is the thin ctypes binding (``q4linear``), the in-tree build (``build``) and
the seeded synthetic workloads (``workloads``).
"""
from .q4linear import (Q4Error, backward_workspace_bytes, dequant,  # noqa: F401
                       library_path, lib, linear, linear_backward, requant,
                       unpack_codes, workspace_bytes)
