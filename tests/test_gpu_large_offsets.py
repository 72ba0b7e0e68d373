"""Tensors past 4 GiB: every entry point at shapes whose byte offsets exceed 32 bits.

A kernel that formed some byte offset in 32 bits would read or write the wrong
rows beyond the first 4 GiB of a tensor, silently. These tests size each tensor
above 4 GiB (many heads of a short sequence for the forward and backward, a
long KV cache for decode) and check heads whose data starts just below, at and
beyond the 4 GiB mark against the FP64 oracle, by the same gates as the other
parity tests. Only the checked heads hold seeded random values; every other
head is zero, which keeps the inputs cheap and gives a closed form to check as
well: zero Q and K make every visible key weigh the same, so a zero head has
O = 0 exactly and lse = ln(number of visible keys), and zero gradients.
"""
import math
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from gpu_helpers import bwd_elem_bounds, check_grad, check_lse, check_o, have_gpu, to_dev, to_f64
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

# 16,500 heads of 1,024 rows x 128 columns: 256 KiB per head in BF16, so head
# 16,384 starts exactly at 4 GiB and the tensor ends at 4.33 GB.
H_BIG, N_BIG, D_BIG = 16500, 1024, 128
HEADS = [0, 8192, 16383, 16384, 16499]     # checked heads (random data)
ZERO_HEADS = [100, 16450]                  # zero heads with a closed-form result


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _scatter_bf16(shape, heads, bits):
    """A zero BF16 tensor of `shape` [1, H, N, d] on the GPU with bits[:, i] placed at head heads[i]."""
    t = torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
    for i, h in enumerate(heads):
        t[:, h] = to_dev(bits[:, i])
    return t


def _check_zero_head_lse(lse_row, causal, n_keys, what):
    """lse of a zero head: ln(i + 1) for causal row i, ln(n_keys) otherwise."""
    n = np.arange(1, lse_row.shape[-1] + 1, dtype=np.float64) if causal else np.full(lse_row.shape, n_keys, np.float64)
    ref = np.log(n)
    rel = float((np.abs(lse_row - ref) / np.maximum(np.abs(ref), 1.0)).max())
    assert rel <= 1e-6, f"{what}: zero-head lse off its closed form by {rel:.3e}"


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_beyond_4gib(causal):
    import exact_tiled_attention_fa_amd as fa
    what = f"fwd 1x{H_BIG}x{N_BIG} d{D_BIG} causal={causal}"
    _say(f"[large] {what} heads={HEADS}")
    case = si.FwdCase("large fwd", 1, len(HEADS), len(HEADS), N_BIG, D_BIG, causal, seed=9100 + int(causal))
    qb, kb, vb = si.fwd_inputs(case)
    shape = (1, H_BIG, N_BIG, D_BIG)
    assert 2 * H_BIG * N_BIG * D_BIG > 2 ** 32
    q, k, v = (_scatter_bf16(shape, HEADS, x) for x in (qb, kb, vb))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_s, lse_s = to_f64(o[:, HEADS]), to_f64(lse[:, HEADS])
    o_z, lse_z = to_f64(o[:, ZERO_HEADS]), to_f64(lse[:, ZERO_HEADS])
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    qf, kf, vf = si.bf16_bits_to_f32(qb), si.bf16_bits_to_f32(kb), si.bf16_bits_to_f32(vb)
    ox_ref, lse_ref = fa_oracle.attention_ref(qf, kf, np.concatenate([vf, np.abs(vf)], axis=-1), causal, case.scale)
    check_o(o_s, ox_ref[..., :D_BIG], ox_ref[..., D_BIG:], what)
    check_lse(lse_s, lse_ref, what)
    assert (o_z == 0).all(), f"{what}: a zero head's O is not 0"
    for j in range(len(ZERO_HEADS)):
        _check_zero_head_lse(lse_z[0, j], causal, N_BIG, what)


def test_fwd_fp8_beyond_4gib():
    """FP8 codes take one byte, so 2,048 rows per head put head 16,384 at 4 GiB."""
    import exact_tiled_attention_fa_amd as fa
    from test_gpu_fwd_fp8 import LSE_REL, U8, _bounds
    from gpu_helpers import ulp_bf16
    N = 2048
    what = f"fwd fp8 1x{H_BIG}x{N} d{D_BIG} causal"
    _say(f"[large] {what} heads={HEADS}")
    case = si.FwdCase("large fp8", 1, len(HEADS), len(HEADS), N, D_BIG, True, seed=9200)
    q8, k8, v8, qs, ks, vs = si.fwd_fp8_inputs(case)
    assert H_BIG * N * D_BIG > 2 ** 32

    def scatter(codes):
        t = torch.zeros((1, H_BIG, N, D_BIG), dtype=torch.uint8, device="cuda:0")
        for i, h in enumerate(HEADS):
            t[:, h] = torch.from_numpy(np.ascontiguousarray(codes[:, i])).to("cuda:0")
        return t.view(torch.float8_e4m3fn)

    q, k, v = scatter(q8), scatter(k8), scatter(v8)
    o, lse = fa.fwd_fp8(q, k, v, qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    o_s, lse_s = to_f64(o[:, HEADS]), to_f64(lse[:, HEADS])
    o_z, lse_z = to_f64(o[:, ZERO_HEADS]), to_f64(lse[:, ZERO_HEADS])
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    o_ref, lse_ref, p = fa_oracle.attention_fp8_ref(q8, k8, v8, qs, ks, vs, True, case.scale, return_p=True)
    bound = _bounds(q8, k8, v8, qs, ks, vs, True, case.scale, None, o_ref, p, False)
    del p
    full = bound + 0.5 * ulp_bf16(np.abs(o_ref) * (1 + 2.0 ** -7)) + 1e-6
    err = np.abs(o_s - o_ref)
    ratio = float((err / full).max())
    rel_rms = float(np.sqrt((err ** 2).sum() / (o_ref ** 2).sum()))
    lse_rel = float((np.abs(lse_s - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)).max())
    _say(f"    {what}: elem_ratio {ratio:.3f} rel_rms {rel_rms:.3e} lse_rel {lse_rel:.3e}")
    assert np.isfinite(o_s).all() and ratio <= 1.0 and rel_rms <= U8 and lse_rel <= LSE_REL
    assert (o_z == 0).all(), f"{what}: a zero head's O is not 0"
    for j in range(len(ZERO_HEADS)):
        _check_zero_head_lse(lse_z[0, j], True, N, what)


@pytest.mark.parametrize("varlen", [False, True], ids=["uniform", "varlen"])
def test_decode_beyond_4gib(varlen):
    """KV caches of 1,100,003 keys: sequence 1's last KV head spans 4.22-4.51 GB of each cache tensor."""
    import exact_tiled_attention_fa_amd as fa
    B, Hq, Hkv, L, d, splits = 2, 32, 8, 1_100_003, 128, 16
    G = Hq // Hkv
    slices = [(0, 0), (1, Hkv - 1)]            # (sequence, KV head) with random data
    zero = (1, 3)                              # a zero slice: O = 0, lse = ln(keys)
    lens = [L, L - 5]
    what = f"decode B{B} Hq{Hq} Hkv{Hkv} L{L} varlen={varlen}"
    _say(f"[large] {what} slices={slices}")
    assert 2 * B * Hkv * L * d > 2 ** 32
    rng = np.random.default_rng(9300)
    qb = si.normal_bf16(rng, (B, Hq, 1, d))
    kv_bits = {s: (si.normal_bf16(rng, (L, d)), si.normal_bf16(rng, (L, d))) for s in slices}
    k = torch.zeros((B, Hkv, L, d), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros_like(k)
    for (b, hk), (kb, vb) in kv_bits.items():
        k[b, hk] = to_dev(kb)
        v[b, hk] = to_dev(vb)
    q = to_dev(qb)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda:0") if varlen else None
    o, lse = fa.decode(q, k, v, num_splits=splits, seq_lens=lens_t)
    torch.cuda.synchronize()
    o_np, lse_np = to_f64(o)[:, :, 0], to_f64(lse)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    scale = d ** -0.5
    qf = si.bf16_bits_to_f32(qb)
    for (b, hk), (kb, vb) in kv_bits.items():
        hs = slice(hk * G, (hk + 1) * G)
        kf = si.bf16_bits_to_f32(kb)[None, None]
        vf = si.bf16_bits_to_f32(vb)[None, None]
        vx = np.concatenate([vf, np.abs(vf)], axis=-1)
        if varlen:
            ox, lse_ref = fa_oracle.decode_varlen_ref(qf[b:b + 1, hs], kf, vx, [lens[b]], scale)
        else:
            ox, lse_ref = fa_oracle.decode_ref(qf[b:b + 1, hs], kf, vx, scale)
        ox = ox.reshape(1, G, 2 * d)
        check_o(o_np[b:b + 1, hs], ox[..., :d], ox[..., d:], f"{what} slice {(b, hk)}")
        check_lse(lse_np[b:b + 1, hs], lse_ref.reshape(1, G), f"{what} slice {(b, hk)}")
    b, hk = zero
    n_keys = lens[b] if varlen else L
    assert (o_np[b, hk * G:(hk + 1) * G] == 0).all(), f"{what}: the zero slice's O is not 0"
    ref = math.log(n_keys)
    rel = float(np.abs(lse_np[b, hk * G:(hk + 1) * G] - ref).max()) / ref
    assert rel <= 1e-6, f"{what}: zero-slice lse off ln(keys) by {rel:.3e}"


def test_bwd_beyond_4gib():
    import exact_tiled_attention_fa_amd as fa
    heads = [0, 16383, 16384, 16499]
    what = f"bwd 1x{H_BIG}x{N_BIG} d{D_BIG} causal"
    _say(f"[large] {what} heads={heads}")
    case = si.FwdCase("large bwd", 1, len(heads), len(heads), N_BIG, D_BIG, True, seed=9400)
    qb, kb, vb = si.fwd_inputs(case)
    gb = si.normal_bf16(np.random.default_rng(9401), (1, len(heads), N_BIG, D_BIG))
    shape = (1, H_BIG, N_BIG, D_BIG)
    q, k, v, g = (_scatter_bf16(shape, heads, x) for x in (qb, kb, vb, gb))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    got = [to_f64(x[:, heads]) for x in (dq, dk, dv)]
    zeros = [to_f64(x[:, ZERO_HEADS]) for x in (dq, dk, dv)]
    del q, k, v, g, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    qf, kf, vf, gf = (si.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb, gb))
    refs = fa_oracle.attention_bwd_ref(qf, kf, vf, gf, True, case.scale)
    bounds = bwd_elem_bounds(qf, kf, vf, gf, True, case.scale)
    for name, x, ref, bnd in zip(("dq", "dk", "dv"), got, refs, bounds):
        check_grad(name, x, ref, bnd, what)
    for name, z in zip(("dq", "dk", "dv"), zeros):
        assert (z == 0).all(), f"{what}: a zero head's {name} is not 0"
