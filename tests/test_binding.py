"""The Python binding rejects tensors too small for the sizes it passes to
the C ABI (which sees pitches, not extents) with ValueError, before any
device check and before anything is queued.  CPU tensors suffice: the
extent checks run first."""
import pytest
import torch

from bit_weight_only_int4_amd import q4linear as b

M, K, N, GS = 4, 256, 128, 32


def t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def good():
    return dict(x=t(M, K), qw=t(N, K // 2, dtype=torch.uint8), scales=t(K // GS, N),
                bias=t(N), out=t(M, N))


@pytest.mark.parametrize("name,bad,match", [
    ("x", t(M, K - 1), "fewer than K"),
    ("x", t(K), "2-D"),
    ("qw", t(N, K // 2 - 1, dtype=torch.uint8), r"ceil\(K / 2\)"),
    ("scales", t(K // GS - 1, N), "grouped scales"),
    ("scales", t(K // GS, N - 1), "grouped scales"),
    ("bias", t(N - 1), "bias needs"),
    ("out", t(1, N), "out must be"),
    ("out", t(M, N + 1), "out must be"),
])
@pytest.mark.parametrize("fn", ["linear", "linear_noalloc"])
def test_linear_rejects_undersized_tensors(fn, name, bad, match):
    a = good()
    a[name] = bad
    with pytest.raises(ValueError, match=match):
        getattr(b, fn)(a["x"], a["qw"], a["scales"], a["bias"], out=a["out"], K=K,
                       group_size=GS)


def test_per_channel_scales_need_n_entries():
    a = good()
    with pytest.raises(ValueError, match="per-channel scales"):
        b.linear(a["x"], a["qw"], t(N - 1), None, K=K, group_size=0)


def test_extents_are_checked_before_the_device():
    # right extents on the CPU: the next check is the device one
    a = good()
    with pytest.raises(ValueError, match="device"):
        b.linear(a["x"], a["qw"], a["scales"], a["bias"], out=a["out"], K=K, group_size=GS)


def test_backward_rejects_undersized_tensors():
    qw, s = t(N, K // 2, dtype=torch.uint8), t(K // GS, N)
    with pytest.raises(ValueError, match="dx must be"):
        b.linear_backward(t(M, N), qw, s, K=K, group_size=GS, dx=t(M - 1, K))
    with pytest.raises(ValueError, match="qw"):
        b.linear_backward(t(M, N), t(N, K // 2 - 1, dtype=torch.uint8), s, K=K, group_size=GS)
    with pytest.raises(ValueError, match="grouped scales"):
        b.linear_backward(t(M, N), qw, t(K // GS - 1, N), K=K, group_size=GS)


def test_requant_unpack_dequant_reject_undersized_tensors():
    with pytest.raises(ValueError, match="qw must be"):
        b.requant(t(N, K), t(K // GS, N), group_size=GS, qw=t(N, K // 2 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="grouped scales"):
        b.requant(t(N, K), t(K // GS, N - 1), group_size=GS)
    with pytest.raises(ValueError, match=r"ceil\(K / 2\)"):
        b.unpack_codes(t(N, K // 2 - 1, dtype=torch.uint8), K)
    with pytest.raises(ValueError, match="per-channel scales"):
        b.dequant(t(N, K // 2, dtype=torch.uint8), t(N - 1), K, 0)


def test_binding_refuses_a_library_built_from_other_sources(monkeypatch):
    """The in-tree library carries a digest of the sources it was built from;
    a library whose digest differs from the tree's is refused, not run."""
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b._build, "source_digest", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="does not match the sources"):
        b.lib()
    monkeypatch.setattr(b, "_lib", None)


def test_in_tree_library_stamp_matches_sources():
    assert b._build.stale_reason(b._build.TREE_LIB) is None


def test_oracle_loader_refuses_a_stale_library(monkeypatch):
    from oracle import build as obuild
    from oracle import q4_oracle as orc
    assert obuild.stale_reason(obuild.TREE_LIB) is None
    monkeypatch.setattr(orc, "_lib", None)
    monkeypatch.setattr(obuild, "source_digest", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="does not match q4_oracle.c"):
        orc._load()
    monkeypatch.setattr(orc, "_lib", None)
