"""The C ABI on the host: the library loads, exports every function that
include/q4linear.h declares, and rejects every invalid argument with its
status code before queueing anything.

No compute call is made here: every call either fails a check or is the
M == 0 / N == 0 no-op, so the pointers below are never dereferenced (they
are placeholders, distinct and far apart).
"""
import ctypes
import os
import re

import pytest

from bit_weight_only_int4_amd import q4linear as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "q4linear.h")

OK, INVALID, ALIAS, WORKSPACE = 0, 1, 2, 3

X, Q, S, BIAS, OUT, WS = (0x10000000, 0x20000000, 0x30000000, 0x40000000,
                          0x50000000, 0x60000000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(q4_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(b.SYMBOLS), names
    L = b.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.q4_abi_version() == b.ABI_VERSION
    for code, text in b.STATUS.items():
        assert L.q4_status_str(code).decode() == text


def base_args(**kw):
    a = dict(x=X, ldx=256, qw=Q, ldq=128, scales=S, lds=128, gs=32, bias=BIAS, out=OUT,
             ldo=128, M=4, N=128, K=256, order=0, math=0, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return a


def call(a):
    path = ctypes.c_int32(-1)
    st = b.lib().q4_linear(a["x"], a["ldx"], a["qw"], a["ldq"], a["scales"], a["lds"],
                           a["gs"], a["bias"], a["out"], a["ldo"], a["M"], a["N"], a["K"],
                           a["order"], a["math"], a["ws"], a["ws_bytes"], a["stream"],
                           ctypes.byref(path))
    return st, path.value


@pytest.mark.parametrize("field,value", [
    ("x", None), ("qw", None), ("scales", None), ("out", None),
    ("M", -1), ("N", -1), ("K", 0), ("K", -5), ("gs", -1),
    ("ldx", 255), ("ldq", 127), ("lds", 127), ("ldo", 127),
    ("order", 2), ("order", -1), ("math", 4), ("math", -1),
    ("x", X + 2), ("out", OUT + 1), ("scales", S + 3), ("bias", BIAS + 2),
    ("M", 1 << 31), ("N", 1 << 31), ("K", 1 << 31),
])
def test_invalid_arguments(field, value):
    st, path = call(base_args(**{field: value}))
    assert st == INVALID
    assert path == 0


def test_odd_k_packed_pitch():
    # K = 255 needs ceil(255 / 2) = 128 bytes per row
    assert call(base_args(K=255, ldq=127, ldx=255))[0] == INVALID
    # per-channel scales do not need lds >= N
    assert call(base_args(gs=0, lds=0, ldx=255, K=255, ldq=127))[0] == INVALID


@pytest.mark.parametrize("out", [X, X + 4 * 100, Q + 64, S, BIAS])
def test_output_overlapping_an_input_is_rejected(out):
    st, _ = call(base_args(out=out))
    assert st == ALIAS


def test_noops_are_ok_and_queue_nothing():
    for M, N in ((0, 128), (4, 0), (0, 0)):
        st, path = call(base_args(M=M, N=N, x=None, qw=None, out=None, scales=None))
        assert st == OK and path == 0


def test_workspace_is_required_when_the_plan_splits():
    L = b.lib()
    # a tall-K, narrow-N decode is split over K
    M, N, K = 1, 64, 65536
    need = L.q4_linear_workspace_bytes(M, N, K, 32, 0)
    assert need > 0
    a = base_args(M=M, N=N, K=K, ldx=K, ldq=K // 2, lds=N, ldo=N)
    assert call(a)[0] == WORKSPACE
    a.update(ws=WS, ws_bytes=need - 4)
    assert call(a)[0] == WORKSPACE
    a.update(ws=OUT, ws_bytes=need)
    assert call(a)[0] == ALIAS


# (M, K, N, group_size, runs an fp32 GEMV): the automatic choice at and
# around the boundaries of its rule.  Shapes of the few-row MFMA kernel
# (K % 32 == 0, per-channel or power-of-two groups >= 32): fp32 only for
# M <= 4 with N*K <= 2^22 or M == 2 with N*K <= 2^25.  Other shapes: fp32 for
# M <= 16 with M*N*K <= 2^26 or M == 2 with M*N*K <= 2^30 (staged or
# per-channel scales, K % 4 == 0).
REGIME = [
    (1, 2048, 128257, 0, True), (1, 14336, 4096, 128, True),
    (4, 2048, 2048, 32, True), (4, 2048, 2049, 32, False), (5, 2048, 2048, 32, False),
    (4, 2048, 300, 32, True), (3, 4096, 1024, 0, True), (3, 4096, 1025, 0, False),
    (2, 2048, 16384, 32, True), (2, 2048, 16385, 32, False), (2, 2048, 128257, 0, False),
    (3, 2048, 128257, 0, False), (32, 2048, 64, 32, False),
    (16, 2040, 2048, 32, True), (16, 2040, 2100, 32, False), (17, 2040, 64, 32, False),
    (2, 2040, 263100, 0, True), (2, 2040, 263200, 0, False),
    (4, 2048, 300, 8, False), (4, 2046, 300, 0, False), (4, 2048, 300, 48, False),
    (4, 2040, 300, 32, True),
]


@pytest.mark.parametrize("M,K,N,gs,gemv", REGIME)
def test_automatic_regime_from_sizes(M, K, N, gs, gemv):
    """The automatic choice depends on sizes alone.  Below 16384 k the fp32
    kernels need no workspace while the MFMA GEMM always does (its binary16
    activations), so the workspace query shows which one a call runs; an
    explicit math overrides the choice."""
    L = b.lib()
    assert (L.q4_linear_workspace_bytes(M, N, K, gs, 0) == 0) == gemv
    assert L.q4_linear_workspace_bytes(M, N, K, gs, 1) == 0
    assert L.q4_linear_workspace_bytes(M, N, K, gs, 2) > 0


def test_workspace_query_is_zero_for_invalid_sizes():
    L = b.lib()
    assert L.q4_linear_workspace_bytes(-1, 10, 10, 0, 0) == 0
    assert L.q4_linear_workspace_bytes(1, 10, 0, 0, 0) == 0


def test_stage_exports_validate():
    L = b.lib()
    codes = 0x70000000
    assert L.q4_unpack_codes(Q, 127, 16, 255, 0, codes, 255, None) == INVALID
    assert L.q4_unpack_codes(Q, 128, 16, 255, 0, codes, 254, None) == INVALID
    assert L.q4_unpack_codes(Q, 128, 16, 255, 3, codes, 255, None) == INVALID
    assert L.q4_unpack_codes(Q, 128, 16, 255, 0, None, 255, None) == INVALID
    assert L.q4_unpack_codes(Q, 128, 16, 255, 0, Q + 8, 255, None) == ALIAS
    assert L.q4_unpack_codes(Q, 128, 0, 255, 0, codes, 255, None) == OK
    w = 0x70000000
    assert L.q4_dequant(Q, 128, S, 16, 32, 16, 255, 0, 2, w, 255, None) == INVALID
    assert L.q4_dequant(Q, 128, S, 15, 32, 16, 255, 0, 0, w, 255, None) == INVALID
    assert L.q4_dequant(Q, 128, S, 16, 32, 16, 255, 0, 1, w + 1, 255, None) == INVALID
    assert L.q4_dequant(Q, 128, S, 16, 32, 16, 255, 0, 0, S + 4, 255, None) == ALIAS
    assert L.q4_dequant(Q, 128, S, 16, 32, 0, 255, 0, 0, w, 255, None) == OK


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(b._build, "LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        b.lib()


def test_backward_and_requant_validate():
    """Argument checks of q4_linear_backward and q4_requant (no compute)."""
    L = b.lib()
    DO, DX, LAT = 0x70000000, 0x80000000, 0x90000000
    path = ctypes.c_int32(-1)

    def bwd(**kw):
        a = dict(dout=DO, lddo=128, qw=Q, ldq=128, scales=S, lds=128, gs=32, dx=DX,
                 lddx=256, M=2, N=128, K=256, order=0, math=0, ws=None, ws_bytes=0)
        a.update(kw)
        return L.q4_linear_backward(a["dout"], a["lddo"], a["qw"], a["ldq"], a["scales"],
                                    a["lds"], a["gs"], a["dx"], a["lddx"], a["M"], a["N"],
                                    a["K"], a["order"], a["math"], a["ws"], a["ws_bytes"],
                                    None, ctypes.byref(path))
    for kw in (dict(dout=None), dict(dx=None), dict(qw=None), dict(scales=None),
               dict(M=-1), dict(N=0), dict(K=0), dict(gs=-1), dict(lddo=127),
               dict(ldq=127), dict(lds=127), dict(lddx=255), dict(order=2), dict(math=5),
               dict(dout=DO + 2), dict(dx=DX + 1)):
        assert bwd(**kw) == INVALID, kw
    # the MFMA backward needs one scale per packed word, and always a workspace
    # (binary16 dout)
    assert bwd(math=2, gs=3, lds=128) == 4
    assert bwd(math=2, gs=20) == 4
    assert bwd(math=2) == WORKSPACE
    assert L.q4_linear_backward_workspace_bytes(2, 128, 256, 32, 2) >= 128 * 128 * 2
    for dx in (DO, Q + 8, S):
        assert bwd(dx=dx) == ALIAS
    assert bwd(M=0, dout=None, dx=None) == OK
    # one block of weight rows needs no workspace; several do
    assert L.q4_linear_backward_workspace_bytes(2, 128, 256, 32, 0) == 0
    assert L.q4_linear_backward_workspace_bytes(2, 1024, 256, 32, 0) > 0
    assert bwd(N=1024, lddo=1024, lds=1024) == WORKSPACE

    def rq(**kw):
        a = dict(lat=LAT, ldl=256, scales=S, lds=128, gs=32, N=128, K=256, order=0, qw=Q,
                 ldq=128)
        a.update(kw)
        return L.q4_requant(a["lat"], a["ldl"], a["scales"], a["lds"], a["gs"], a["N"],
                            a["K"], a["order"], a["qw"], a["ldq"], None)
    for kw in (dict(lat=None), dict(scales=None), dict(qw=None), dict(N=-1), dict(K=0),
               dict(ldl=255), dict(ldq=127), dict(lds=127), dict(gs=-1), dict(order=2),
               dict(lat=LAT + 2)):
        assert rq(**kw) == INVALID, kw
    assert rq(qw=LAT + 64) == ALIAS and rq(qw=S + 4) == ALIAS
    assert rq(N=0, lat=None, qw=None, scales=None) == OK


def test_f16_scale_entry_validates():
    """q4_linear_f16_scales: the checks of q4_linear, with 2-byte scale
    elements (alignment and the aliasing range follow the element size)."""
    def call16(**kw):
        a = base_args(**kw)
        path = ctypes.c_int32(-1)
        st = b.lib().q4_linear_f16_scales(
            a["x"], a["ldx"], a["qw"], a["ldq"], a["scales"], a["lds"], a["gs"], a["bias"],
            a["out"], a["ldo"], a["M"], a["N"], a["K"], a["order"], a["math"], a["ws"],
            a["ws_bytes"], a["stream"], ctypes.byref(path))
        return st, path.value
    for kw in (dict(scales=None), dict(scales=S + 1), dict(lds=127), dict(K=0),
               dict(order=2), dict(math=5), dict(x=X + 2)):
        assert call16(**kw) == (INVALID, 0), kw
    # 8 groups x 128 binary16 scales end 2048 bytes after S
    assert call16(out=S + 2044)[0] == ALIAS
    assert call16(M=0, scales=None, x=None, qw=None, out=None) == (OK, 0)


def call_noalloc(a):
    path = ctypes.c_int32(-1)
    st = b.lib().q4_linear_noalloc(a["x"], a["ldx"], a["qw"], a["ldq"], a["scales"], a["lds"],
                                   a["gs"], a["bias"], a["out"], a["ldo"], a["M"], a["N"],
                                   a["K"], a["order"], a["math"], a["stream"],
                                   ctypes.byref(path))
    return st, path.value


@pytest.mark.parametrize("field,value", [
    ("x", None), ("out", None), ("M", -1), ("K", 0), ("ldx", 255), ("order", 2), ("math", 4),
])
def test_noalloc_invalid_arguments(field, value):
    # invalid sizes need no workspace, so q4_linear's checks report them
    a = base_args(M=1)
    a[field] = value
    st, path = call_noalloc(a)
    assert st == INVALID
    assert path == 0


def test_noalloc_rejects_workspace_beyond_its_array():
    # 2048 x 32768 binary16 activations alone exceed the 64 MiB array: the
    # call stops before looking up any device
    need = b.lib().q4_linear_workspace_bytes(2048, 256, 32768, 32, 0)
    assert need > b.NOALLOC_SCRATCH_BYTES
    st, path = call_noalloc(base_args(M=2048, N=256, K=32768, ldx=32768, ldq=16384, lds=256,
                                      ldo=256, bias=None))
    assert st == WORKSPACE
    assert path == 0


def test_noalloc_empty_is_a_no_op():
    assert call_noalloc(base_args(M=0))[0] == OK
    assert call_noalloc(base_args(N=0))[0] == OK


UNSUPPORTED = 4


def test_bf16_math_is_unsupported_everywhere():
    """Q4_MATH_BF16 is a valid request that is not built: every entry point
    taking a math rejects it with Q4_ERR_UNSUPPORTED before queueing
    anything, also for empty sizes; its workspace query is 0."""
    L = b.lib()
    assert call(base_args(math=3)) == (UNSUPPORTED, 0)
    assert call(base_args(math=3, M=0)) == (UNSUPPORTED, 0)
    assert call_noalloc(base_args(math=3)) == (UNSUPPORTED, 0)
    assert L.q4_linear_workspace_bytes(4, 128, 256, 32, 3) == 0
    path = ctypes.c_int32(-1)
    st = L.q4_linear_f16_scales(X, 256, Q, 128, S, 128, 32, BIAS, OUT, 128, 4, 128, 256, 0, 3,
                                None, 0, None, ctypes.byref(path))
    assert (st, path.value) == (UNSUPPORTED, 0)
    st = L.q4_linear_backward(0x70000000, 128, Q, 128, S, 128, 32, 0x80000000, 256, 2, 128,
                              256, 0, 3, None, 0, None, ctypes.byref(path))
    assert (st, path.value) == (UNSUPPORTED, 0)
    assert L.q4_linear_backward_workspace_bytes(2, 128, 256, 32, 3) == 0


def test_workspace_must_be_16_byte_aligned():
    L = b.lib()
    M, N, K = 1, 64, 65536
    need = L.q4_linear_workspace_bytes(M, N, K, 32, 0)
    a = base_args(M=M, N=N, K=K, ldx=K, ldq=K // 2, lds=N, ldo=N)
    for off in (4, 8, 12):
        a.update(ws=WS + off, ws_bytes=need + 64)
        assert call(a)[0] == WORKSPACE, off
