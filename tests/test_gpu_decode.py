"""GPU parity of split-KV decode (split kernel + combine) against the FP64 oracle."""
import sys

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import check_lse, check_o, have_gpu, to_dev, to_f64
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _run(case: si.DecodeCase, scale=None, check_partials=False):
    import torch
    import exact_tiled_attention_fa_amd as fa
    scale = case.scale if scale is None else scale
    print(f"[decode] {case.name} seed={case.seed} scale={scale}", flush=True)
    sys.stdout.flush()
    qb, kb, vb = si.decode_inputs(case)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    need = fa.decode_workspace_bytes(case.B, case.Hq, case.L, case.d, case.num_splits)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")  # stale contents must not matter
    o, lse = fa.decode(q, k, v, num_splits=case.num_splits, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    qf, kf, vf = si.bf16_bits_to_f32(qb), si.bf16_bits_to_f32(kb), si.bf16_bits_to_f32(vb)
    ox_ref, lse_ref = fa_oracle.decode_ref(qf, kf, np.concatenate([vf, np.abs(vf)], axis=-1), scale)
    o_ref, pabs_ref = ox_ref[..., :case.d], ox_ref[..., case.d:]
    stats = check_o(to_f64(o)[:, :, 0], o_ref, pabs_ref, case.name, flat_gate=abs(scale - case.scale) < 1e-12)
    stats["lse_rel"] = check_lse(to_f64(lse), lse_ref, case.name)
    if check_partials:
        chunks = [c for c in fa_oracle.split_chunks(case.L, case.num_splits) if c[1] > c[0]]
        S = len(chunks)
        wsf = ws.view(torch.float32)
        n_o = case.B * case.Hq * S * case.d
        op = to_f64(wsf[:n_o]).reshape(case.B, case.Hq, S, case.d)
        lp = to_f64(wsf[n_o:n_o + case.B * case.Hq * S]).reshape(case.B, case.Hq, S)
        op_ref, lp_ref = fa_oracle.split_decode_partials_ref(qf, kf, vf, scale, case.num_splits)
        # FP32 partials: tight element-wise agreement.
        assert np.max(np.abs(op - op_ref[:, :, :S])) < 1e-4
        assert np.max(np.abs(lp - lp_ref[:, :, :S]) / np.maximum(np.abs(lp_ref[:, :, :S]), 1)) < 1e-5
    return stats


def test_decode_gqa_workload():
    _run(si.DECODE_GQA, check_partials=True)


@pytest.mark.parametrize("L,splits", [(1000, 16), (5, 4), (1, 1), (130, 130), (4097, 3), (8192, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_ragged_splits(L, splits, d):
    _run(si.DecodeCase(f"L{L} s{splits} d{d}", 2, 8, 2, L, d, splits, seed=200 + L + d), check_partials=True)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 3), (8, 1), (24, 3), (32, 1), (40, 2)])
def test_decode_group_sizes(Hq, Hkv):
    _run(si.DecodeCase(f"G{Hq // Hkv}", 3, Hq, Hkv, 777, 128, 5, seed=300 + Hq))


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_decode_scale_edge_cases(scale):
    _run(si.DecodeCase("scale", 2, 8, 2, 600, 128, 7, seed=400), scale=scale)


def _run_varlen(name, B, Hq, Hkv, L, d, splits, lens, seed):
    """Variable-length decode: padding rows hold NaN, which any read of them
    would carry into the output; empty sequences must give O = 0, lse = -inf."""
    import torch
    import exact_tiled_attention_fa_amd as fa
    case = si.DecodeCase(name, B, Hq, Hkv, L, d, splits, seed=seed)
    print(f"[decode-varlen] {name} seed={seed} lens={list(lens)}", flush=True)
    sys.stdout.flush()
    qb, kb, vb = si.decode_inputs(case)
    nan = np.uint16(0x7FC0)  # BF16 quiet NaN
    n_eff = np.clip(np.asarray(lens), 0, L)
    for b, n in enumerate(n_eff):
        kb[b, :, n:] = nan
        vb[b, :, n:] = nan
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    lens_t = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda:0")
    need = fa.decode_workspace_bytes(B, Hq, L, d, splits)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")
    o, lse = fa.decode(q, k, v, num_splits=splits, scale=case.scale, workspace=ws, seq_lens=lens_t)
    torch.cuda.synchronize()
    o_np, lse_np = to_f64(o)[:, :, 0], to_f64(lse)
    qf, kf, vf = si.bf16_bits_to_f32(qb), si.bf16_bits_to_f32(kb), si.bf16_bits_to_f32(vb)
    ox_ref, lse_ref = fa_oracle.decode_varlen_ref(qf, kf, np.concatenate([vf, np.abs(vf)], axis=-1), lens, case.scale)
    o_ref, pabs_ref = ox_ref[..., :d], ox_ref[..., d:]
    empty = n_eff == 0
    assert (o_np[empty] == 0).all() and np.isneginf(lse_np[empty]).all()
    if (~empty).any():
        check_o(o_np[~empty], o_ref[~empty], pabs_ref[~empty], name)
        check_lse(lse_np[~empty], lse_ref[~empty], name)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_varlen_edges(d):
    # L = 1000, 8 splits -> chunks of 125 keys: lengths at, around and inside chunk edges,
    # one key, all keys, none, and counts outside [0, L] (clamped).
    lens = [1, 124, 125, 126, 999, 1000, 0, 2000, -5, 377]
    _run_varlen(f"varlen d{d}", len(lens), 8, 2, 1000, d, 8, lens, seed=500 + d)


def test_decode_varlen_workload_shape():
    """The GQA decode workload's shape with seeded random cache lengths."""
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 8193, size=16)
    _run_varlen("varlen B16 Hq32 Hkv8 L8192", 16, 32, 8, 8192, 128, 16, lens, seed=5)
