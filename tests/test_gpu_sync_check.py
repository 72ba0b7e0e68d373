"""Race check: the normal library against its race-check build, bit for bit.

libfa_sync.so is built from the same sources with -DFA_SYNC_CHECK=1: every
phase of a kernel that hands data through LDS, or fills LDS with direct
HBM->LDS loads, ends with a wait for all outstanding memory operations and a
work-group barrier (a wave-level wait where only one wave owns the data), and
the forward kernels issue all of a step's loads before its products. The
arithmetic and its order are unchanged, so every output must match libfa.so
exactly; a read that met a buffer before its data landed, or after another
wave had started to overwrite it, would show up as a difference. Each entry
point also runs twice through libfa.so: the results must be deterministic.

The shapes take each kernel's distinct paths: the single-launch and key-split
forward (uniform and per-block causal splits), four- and eight-wave causal
blocks with ragged tails, GQA, d = 64 and 128, the FP8 forward, uniform and
variable-length decode, and the backward pass's three kernels.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from exact_tiled_attention_fa_amd import _lib
from gpu_helpers import have_gpu, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def libs():
    return _lib.lib(), _lib.open_library(_lib.SYNC_LIB_PATH)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _bits(t: torch.Tensor) -> torch.Tensor:
    """The tensor's bytes as integers, so that equality is bitwise (NaN == NaN, -0 != +0)."""
    return t.contiguous().view(torch.uint8)


def _same(a, b, what, names=("o", "lse")):
    for x, y, name in zip(a, b, names):
        if not torch.equal(_bits(x), _bits(y)):
            n = int((_bits(x) != _bits(y)).sum())
            raise AssertionError(f"{what}: {name} differs in {n} bytes")


def _check(lib, st, what):
    assert st == 0, f"{what}: {lib.fa_status_string(st).decode()}"


def _fwd(lib, q, k, v, causal):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    need = lib.fa_fwd_workspace_bytes(B, Hq, N, d)
    ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device=q.device)
    st = lib.fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                       int(causal), float(d ** -0.5), ws.data_ptr(), need, _stream())
    _check(lib, st, "fa_fwd_ws")
    torch.cuda.synchronize()
    return o, lse


FWD_CASES = [
    # (B, Hq, Hkv, N, d, causal): the paths each takes on a 256-CU part
    (1, 1, 1, 8192, 128, False),    # uniform key split x8 + combine
    (1, 1, 1, 8192, 128, True),     # per-block causal key splits, single-split blocks write O directly
    (1, 16, 16, 8000, 128, True),   # eight-wave causal blocks, ragged last block
    (2, 8, 2, 1000, 64, True),      # four-wave blocks, GQA, ragged tail, d = 64
    (1, 32, 32, 2048, 128, False),  # single launch, head groups
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else ""))
def test_fwd_matches_race_check_build(libs, case):
    B, Hq, Hkv, N, d, causal = case
    print(f"[sync-check] fwd {case}", flush=True)
    sys.stdout.flush()
    fc = si.FwdCase("sync", B, Hq, Hkv, N, d, causal, seed=7100 + N + d)
    q, k, v = (to_dev(x) for x in si.fwd_inputs(fc))
    normal, sync = libs
    a = _fwd(normal, q, k, v, causal)
    b = _fwd(normal, q, k, v, causal)
    c = _fwd(sync, q, k, v, causal)
    assert torch.isfinite(a[0].float()).all() and torch.isfinite(a[1]).all()
    _same(a, b, "libfa twice")
    _same(a, c, "libfa vs race-check build")


@pytest.mark.parametrize("case", [(1, 8, 8, 2048, 128, False), (1, 8, 8, 2048, 128, True),
                                  (2, 4, 2, 1000, 64, True), (1, 1, 1, 8192, 128, False)],
                         ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else ""))
def test_fwd_fp8_matches_race_check_build(libs, case):
    B, Hq, Hkv, N, d, causal = case
    print(f"[sync-check] fwd fp8 {case}", flush=True)
    sys.stdout.flush()
    q8, k8, v8, qs, ks, vs = si.fwd_fp8_inputs(si.FwdCase("sync8", B, Hq, Hkv, N, d, causal, seed=7200 + N + d))
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in (q8, k8, v8))
    normal, sync = libs

    def run(lib):
        o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda:0")
        need = lib.fa_fwd_workspace_bytes(B, Hq, N, d)
        ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda:0")
        st = lib.fa_fwd_fp8_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), qs, ks, vs, o.data_ptr(), lse.data_ptr(),
                               B, Hq, Hkv, N, d, int(causal), float(d ** -0.5), ws.data_ptr(), need, _stream())
        _check(lib, st, "fa_fwd_fp8_ws")
        torch.cuda.synchronize()
        return o, lse

    a, b, c = run(normal), run(normal), run(sync)
    assert torch.isfinite(a[0].float()).all()
    _same(a, b, "libfa twice")
    _same(a, c, "libfa vs race-check build")


@pytest.mark.parametrize("varlen", [False, True], ids=["uniform", "varlen"])
def test_decode_matches_race_check_build(libs, varlen):
    B, Hq, Hkv, L, d, splits = 8, 32, 8, 3000, 128, 16
    print(f"[sync-check] decode varlen={varlen}", flush=True)
    sys.stdout.flush()
    qb, kb, vb = si.decode_inputs(si.DecodeCase("sync-dec", B, Hq, Hkv, L, d, splits, seed=7300))
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    lens = torch.tensor([3000, 1, 187, 2999, 0, 1500, 64, 2048], dtype=torch.int32, device="cuda:0")
    normal, sync = libs

    def run(lib):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda:0")
        need = lib.fa_decode_workspace_bytes(B, Hq, L, d, splits)
        ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda:0")
        head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
        tail = (B, Hq, Hkv, L, d, splits, float(d ** -0.5), ws.data_ptr(), need, _stream())
        if varlen:
            st = lib.fa_decode_varlen(*head, lens.data_ptr(), *tail)
        else:
            st = lib.fa_decode(*head, *tail)
        _check(lib, st, "fa_decode")
        torch.cuda.synchronize()
        return o, lse

    a, b, c = run(normal), run(normal), run(sync)
    _same(a, b, "libfa twice")
    _same(a, c, "libfa vs race-check build")


@pytest.mark.parametrize("case", [(1, 4, 2, 1000, 64, True), (1, 8, 8, 2048, 128, False),
                                  (2, 4, 4, 1100, 128, True)],
                         ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else ""))
def test_bwd_matches_race_check_build(libs, case):
    B, Hq, Hkv, N, d, causal = case
    print(f"[sync-check] bwd {case}", flush=True)
    sys.stdout.flush()
    fc = si.FwdCase("sync-bwd", B, Hq, Hkv, N, d, causal, seed=7400 + N + d)
    q, k, v = (to_dev(x) for x in si.fwd_inputs(fc))
    dout = to_dev(si.normal_bf16(np.random.default_rng(7500 + N), (B, Hq, N, d)))
    normal, sync = libs
    o, lse = _fwd(normal, q, k, v, causal)

    def run(lib):
        dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
        need = lib.fa_bwd_workspace_bytes(B, Hq, N, d)
        ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda:0")
        st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, int(causal),
                        float(d ** -0.5), ws.data_ptr(), need, _stream())
        _check(lib, st, "fa_bwd")
        torch.cuda.synchronize()
        return dq, dk, dv

    a, b, c = run(normal), run(normal), run(sync)
    assert all(torch.isfinite(x.float()).all() for x in a)
    _same(a, b, "libfa twice", ("dq", "dk", "dv"))
    _same(a, c, "libfa vs race-check build", ("dq", "dk", "dv"))


def test_race_check_build_is_a_distinct_library(libs):
    """The two handles are separate builds (not one library loaded twice)."""
    normal, sync = libs
    assert ctypes.cast(normal.fa_fwd, ctypes.c_void_p).value != ctypes.cast(sync.fa_fwd, ctypes.c_void_p).value
