"""The C-ABI library loads, exports every symbol include/fa.h declares, and
rejects bad arguments on the host before any HIP call (safe without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_tiled_attention_fa_amd", "libfa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from exact_tiled_attention_fa_amd import _lib
    return _lib.lib()


def test_header_declares_the_abi():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_decode", "fa_decode_varlen",
                                     "fa_decode_workspace_bytes", "fa_fwd", "fa_fwd_fp8", "fa_fwd_fp8_ws",
                                     "fa_fwd_noalloc", "fa_fwd_noalloc_max_scratch_bytes",
                                     "fa_fwd_workspace_bytes", "fa_fwd_ws", "fa_fwd_ws_timed", "fa_status_string"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_race_check_build_exports_the_same_abi():
    """libfa_sync.so (the -DFA_SYNC_CHECK=1 build the GPU race check compares
    with libfa.so) is built beside it and exports every declared symbol."""
    from exact_tiled_attention_fa_amd import _lib
    sync = _lib.open_library(_lib.SYNC_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(sync, name), name
    assert sync.fa_status_string(-9).decode().startswith("FA_ERR_SCRATCH")
    assert fwd(sync, d=96) == -3  # host checks run before any device work here too


def test_status_strings(lib):
    from exact_tiled_attention_fa_amd import _lib
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_string(code).decode().startswith(name)
    assert lib.fa_status_string(12345) == b"unknown fa_status"


# Fake, 16-byte aligned, never-dereferenced addresses: every call below fails its
# host-side argument checks before touching the device.
P = 0x10000
BAD = 0x10008  # 8-byte aligned only


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128, causal=0, scale=0.125):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=-1), -2), (dict(N=0), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(d=0), -3),
    (dict(Hq=6, Hkv=4), -4),
    (dict(q=BAD), -5), (dict(o=BAD), -5), (dict(lse=P + 2), -5),
    (dict(causal=2), -8), (dict(scale=float("nan")), -8), (dict(scale=float("inf")), -8),
    (dict(B=1 << 20, Hq=1 << 12, N=1 << 20), -2),
    (dict(N=(1 << 30) + 1), -2), (dict(N=(1 << 31) - 1), -2),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status


def fwd_noalloc(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128, causal=0, scale=0.125):
    return lib.fa_fwd_noalloc(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(N=0), -2), (dict(d=80), -3), (dict(Hq=3, Hkv=2), -4),
    (dict(k=BAD), -5), (dict(causal=2), -8), (dict(scale=float("nan")), -8), (dict(N=(1 << 30) + 1), -2),
])
def test_fwd_noalloc_rejects(lib, kw, status):
    assert fwd_noalloc(lib, **kw) == status


def test_fwd_noalloc_scratch_covers_every_plan(lib):
    """The static scratch holds the key-split partials of every shape the planner
    splits (on the CU count the planner sees here: 256 without a GPU)."""
    most = lib.fa_fwd_noalloc_max_scratch_bytes()
    assert most == 34 << 20
    worst = 0
    for heads in range(1, 130):
        for N in list(range(1024, 70000, 256)) + [65280, 8192]:
            for d in (64, 128):
                worst = max(worst, lib.fa_fwd_workspace_bytes(1, heads, N, d))
    assert 0 < worst <= most


def fwd_ws(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128, causal=0, scale=0.125, ws=P, wsb=0):
    return lib.fa_fwd_ws(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(N=0), -2), (dict(d=80), -3), (dict(Hq=3, Hkv=2), -4),
    (dict(v=BAD), -5), (dict(causal=-1), -8), (dict(scale=float("-inf")), -8),
])
def test_fwd_ws_rejects(lib, kw, status):
    assert fwd_ws(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(N=0), -2), (dict(d=80), -3), (dict(Hq=3, Hkv=2), -4),
    (dict(v=BAD), -5), (dict(causal=-1), -8), (dict(scale=float("-inf")), -8),
])
def test_fwd_ws_timed_rejects(lib, kw, status):
    """fa_fwd_ws_timed applies fa_fwd_ws's checks (before any HIP call) and refuses a NULL event."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128, causal=0, scale=0.125, ws=P, wsb=0)
    a.update(kw)
    assert lib.fa_fwd_ws_timed(*a.values(), None, P) == status
    assert lib.fa_fwd_ws_timed(P, P, P, P, P, 1, 1, 1, 128, 128, 0, 0.125, P, 0, None, None) == -1


def test_fwd_workspace_size_rules(lib):
    assert lib.fa_fwd_workspace_bytes(1, 1, 8192, 128) % 256 == 0
    assert lib.fa_fwd_workspace_bytes(0, 1, 128, 128) == 0
    assert lib.fa_fwd_workspace_bytes(1, 1, 128, 96) == 0
    assert lib.fa_fwd_workspace_bytes(1, 1, 960, 128) == 0  # 15 key tiles: never split
    assert lib.fa_fwd_workspace_bytes(1, 1, (1 << 31) - 1, 64) == 0


def dec(lib, q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, L=100, d=128, splits=4, scale=0.1, ws=P, wsb=1 << 30):
    return lib.fa_decode(q, k, v, o, lse, B, Hq, Hkv, L, d, splits, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(L=0), -2), (dict(splits=0), -2), (dict(splits=101), -2), (dict(B=0), -2),
    (dict(d=32), -3), (dict(Hq=6, Hkv=4), -4),
    (dict(k=BAD), -5), (dict(ws=BAD), -5),
    (dict(scale=float("nan")), -8),
    (dict(ws=None), -6), (dict(wsb=16), -6),
    (dict(L=(1 << 31) - 1, splits=(1 << 31) - 1), -2), (dict(L=(1 << 30) + 1, splits=1), -2),
])
def test_decode_rejects(lib, kw, status):
    assert dec(lib, **kw) == status


def dec_varlen(lib, lens=P, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, L=100, d=128, splits=4, scale=0.1, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.fa_decode_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], lens, a["B"], a["Hq"], a["Hkv"], a["L"],
                                a["d"], a["splits"], a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(lens=None), -1), (dict(lens=P + 2), -5), (dict(q=None), -1), (dict(L=0), -2), (dict(d=80), -3),
    (dict(Hq=6, Hkv=4), -4), (dict(v=BAD), -5), (dict(scale=float("nan")), -8), (dict(wsb=16), -6),
])
def test_decode_varlen_rejects(lib, kw, status):
    assert dec_varlen(lib, **kw) == status


def bwd(lib, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, N=300, d=128, causal=0,
        scale=0.1, ws=P, wsb=1 << 30):
    return lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(do=None), -1), (dict(dk=None), -1), (dict(lse=None), -1),
    (dict(N=0), -2), (dict(B=-1), -2), (dict(d=256), -3), (dict(d=96), -3), (dict(Hq=3, Hkv=2), -4),
    (dict(dv=BAD), -5), (dict(do=BAD), -5), (dict(ws=BAD), -5), (dict(causal=3), -8),
    (dict(scale=float("nan")), -8), (dict(ws=None), -6), (dict(wsb=64), -6),
    (dict(N=(1 << 30) + 1), -2),
])
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_workspace_size(lib):
    # two floats per row, rows padded to 64 per head
    assert lib.fa_bwd_workspace_bytes(1, 2, 300, 128) == (2 * 2 * 320 * 4 + 255) // 256 * 256
    assert lib.fa_bwd_workspace_bytes(1, 2, 300, 64) == (2 * 2 * 320 * 4 + 255) // 256 * 256
    assert lib.fa_bwd_workspace_bytes(1, 2, 300, 96) == 0
    assert lib.fa_bwd_workspace_bytes(0, 2, 300, 128) == 0


def test_decode_workspace_size(lib):
    # 16 x 32 rows, 16 chunks of 512 keys, (128 + 1) floats each.
    assert lib.fa_decode_workspace_bytes(16, 32, 8192, 128, 16) == 16 * 32 * 16 * 129 * 4
    # L = 5, 4 splits -> chunk 2 -> 3 non-empty chunks.
    assert lib.fa_decode_workspace_bytes(1, 1, 5, 64, 4) == (3 * 65 * 4 + 255) // 256 * 256
    assert lib.fa_decode_workspace_bytes(1, 1, 5, 64, 6) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 5, 60, 1) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, (1 << 31) - 1, 64, (1 << 31) - 1) == 0


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import exact_tiled_attention_fa_amd as fa
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(x, x, x)


def test_binding_requires_one_gpu_for_every_tensor():
    """A tensor on another GPU or in host memory (lse, workspace, seq_lens included) is refused before any call."""
    torch = pytest.importorskip("torch")
    from types import SimpleNamespace
    import exact_tiled_attention_fa_amd as fa
    g0, g1 = SimpleNamespace(device=torch.device("cuda:0")), SimpleNamespace(device=torch.device("cuda:1"))
    host = SimpleNamespace(device=torch.device("cpu"))
    assert fa._one_device(("q", g0), ("k", g0), ("seq_lens", None)) == torch.device("cuda:0")
    with pytest.raises(ValueError, match="k is on cuda:1"):
        fa._one_device(("q", g0), ("k", g1))
    with pytest.raises(ValueError, match="lse must be on a GPU"):
        fa._one_device(("q", g0), ("lse", host))
    with pytest.raises(ValueError, match="contiguous"):
        fa._check_workspace(torch.zeros(64, dtype=torch.uint8)[::2])


def fwd_fp8(lib, q=P, k=P, v=P, qs=0.01, ks=0.01, vs=0.01, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128,
            causal=0, scale=0.125):
    return lib.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, Hq, Hkv, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(N=-1), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(d=0), -3),
    (dict(Hq=5, Hkv=2), -4),
    (dict(k=BAD), -5), (dict(lse=P + 1), -5),
    (dict(causal=3), -8), (dict(scale=float("nan")), -8),
    (dict(qs=float("inf")), -8), (dict(ks=float("nan")), -8), (dict(vs=float("-inf")), -8),
    (dict(qs=1e30, ks=1e30), -8),   # scale * q_scale * k_scale overflows FP32
    (dict(B=1 << 20, Hq=1 << 12, N=1 << 20), -2),
])
def test_fwd_fp8_rejects(lib, kw, status):
    assert fwd_fp8(lib, **kw) == status


def test_fwd_fp8_ws_rejects(lib):
    args = dict(q=P, k=P, v=P, qs=0.01, ks=0.01, vs=0.01, o=P, lse=P, B=1, Hq=1, Hkv=1, N=128, d=128,
                causal=0, scale=0.125)

    def call(**kw):
        a = dict(args, **kw)
        return lib.fa_fwd_fp8_ws(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"], a["B"],
                                 a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], P, 0, None)
    assert call(q=None) == -1
    assert call(d=96) == -3
    assert call(vs=float("nan")) == -8


def test_binding_refuses_ints_that_do_not_fit(lib):
    # ctypes would keep the low 32 bits of 2**32 + 128 (i.e. 128); the loader raises instead.
    # Each call also carries a NULL q, so none could reach a launch.
    with pytest.raises(ctypes.ArgumentError):
        lib.fa_fwd_workspace_bytes(1, 1, (1 << 32) + 128, 128)
    with pytest.raises(ctypes.ArgumentError):
        lib.fa_decode_workspace_bytes(1, 1, 100, 128, -(1 << 31) - 1)
    with pytest.raises(ctypes.ArgumentError):
        lib.fa_fwd_workspace_bytes(1, 1, 128.0, 128)
    with pytest.raises(ctypes.ArgumentError):  # negative size_t would wrap to a huge workspace
        lib.fa_fwd_ws(None, P, P, P, P, 1, 1, 1, 128, 128, 0, 0.1, P, -1, None)
    assert fwd_ws(lib, q=None, wsb=(1 << 64) - 1) == -1


def test_missing_library_raises(monkeypatch):
    """No fallback path: without libfa.so every entry point raises."""
    from exact_tiled_attention_fa_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libfa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
