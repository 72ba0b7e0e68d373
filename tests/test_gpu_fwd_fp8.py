"""GPU parity of the FP8 forward pass against the FP64 oracle, through the C ABI.

Inputs: seeded N(0,1) draws quantised per tensor to OCP E4M3 codes
(seeded_inputs.fwd_fp8_inputs / quantize_fp8); the same codes reach the GPU and
the oracle, which decodes them and takes the exact attention of the
dequantised values (attention_fp8_ref).

Tolerances, derived from the kernel's arithmetic (u8 = 2^-4, the relative
half-step of a 3-bit significand):
  * O, element-wise. The kernel forms O_i = v_scale sum_j e4m3(p_ij) V_j / l_i
    with p_ij = 2^(t_ij - m + 6) in FP32 and l_i = sum_j p_ij. With m at most 2
    below the row max, p sits in [2^6, 2^8] times its share of the max, so
    rounding to E4M3 moves it by at most u8 p (normal codes) or by 2^-10 in
    that scale, 2^-16 of the max weight (subnormal codes). In normalised
    weights P_ij that is E_ij = max(u8 P_ij, min(P_ij, 2^-16 max_j P_ij)), and
        |O_gpu - O_ref|_i <= sum_j E_ij |v_j| + eps_i ((P|V|)_i + |O_i|)
                             + 0.5 ulp_bf16(|O_i| (1 + 2^-7)) + 1e-6,
    where eps_i bounds the score error of the FP8 matrix products, which do
    not accumulate at FP32 precision: over 256 random 32x32x64 products of
    E4M3 codes the worst error of v_mfma_f32_32x32x64_f8f6f4 was 2^-14.6 of
    the sum of |products| of the step, so eps_i = 2^-13 |scale q_scale k_scale|
    max_j sum_k |Q8_ik K8_jk| (natural-log units; a score error moves each
    weight by that factor, and the weights' normalisation by the same).
  * O, aggregate: relative RMS error <= u8. For zero-mean i.i.d. values the
    rounding errors are independent of V, so E|dO|^2 / E|O|^2 <= u8^2.
  * lse: |dlse| / max(|lse|, 1) <= 1e-3 (the BF16 pass's gate): the weights'
    rounding does not reach lse (l sums the FP32 values), the score error does,
    at most eps_i.
  * key splits round each split's normalised partial to BF16 before the
    combine: at most 2^-8 (P|V|)_i more (as for the BF16 pass).
"""
import math
import sys

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import LSE_REL, have_gpu, ulp_bf16
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

U8 = 2.0 ** -4
MFMA_F8_REL = 2.0 ** -13  # ~3x the measured worst case, per 64-term step, of the sum of |products|


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(codes):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to("cuda:0")
    return t.view(torch.float8_e4m3fn)


def _bounds(q8, k8, v8, qs, ks, vs, causal, scale, rows, o_ref, p, split):
    """Element bound (without the output rounding) for O at the checked rows;
    with key splits the BF16 rounding of the partials adds 2^-8 (P|V|)."""
    B, Hq, R, N = p.shape
    Hkv = k8.shape[1]
    G = Hq // Hkv
    qv = np.abs(fa_oracle.fp8_e4m3_value(q8))
    kv = np.abs(fa_oracle.fp8_e4m3_value(k8))
    vabs = np.abs(fa_oracle.fp8_e4m3_value(v8) * vs)
    out = np.zeros(o_ref.shape)
    for b in range(B):
        for h in range(Hq):
            ph = p[b, h]
            ids = np.arange(q8.shape[2]) if rows is None else rows[h]
            e = np.maximum(U8 * ph, np.minimum(ph, 2.0 ** -16 * ph.max(axis=1, keepdims=True)))
            va = vabs[b, h // G]
            sabs = qv[b, h, ids] @ kv[b, h // G].T                       # [R, N]
            if causal:
                sabs = np.where(np.arange(N)[None, :] <= ids[:, None], sabs, 0.0)
            eps = MFMA_F8_REL * abs(scale * qs * ks) * sabs.max(axis=1)
            pva = ph @ va
            out[b, h] = e @ va + eps[:, None] * (pva + np.abs(o_ref[b, h])) + (2.0 ** -8 if split else 0.0) * pva
    return out


def _run(name, B, Hq, Hkv, N, causal, seed, scale=None, sampled=None, q_sign=1.0, d=128, codes=None):
    import torch
    import exact_tiled_attention_fa_amd as fa
    case = si.FwdCase(name, B, Hq, Hkv, N, d, causal, seed)
    scale = case.scale if scale is None else scale
    _say(f"[fp8] {name} B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal} seed={seed} scale={scale}")
    q8, k8, v8, qs, ks, vs = si.fwd_fp8_inputs(case) if codes is None else codes
    qs *= q_sign
    q, k, v = _upload(q8), _upload(k8), _upload(v8)
    o, lse = fa.fwd_fp8(q, k, v, qs, ks, vs, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_np = o.to("cpu", torch.float64).numpy()
    lse_np = lse.to("cpu", torch.float64).numpy()
    del q, k, v, o, lse
    rows = None
    if sampled:
        rows = np.stack([si.sample_rows(seed, h, N, sampled) for h in range(Hq)])
        o_np = np.stack([o_np[:, h, rows[h]] for h in range(Hq)], axis=1)
        lse_np = np.stack([lse_np[:, h, rows[h]] for h in range(Hq)], axis=1)
    o_ref, lse_ref, p = fa_oracle.attention_fp8_ref(q8, k8, v8, qs, ks, vs, causal, scale, rows=rows,
                                                    return_p=True)
    split = fa.fwd_workspace_bytes(B, Hq, N, d) > 0
    bound = _bounds(q8, k8, v8, qs, ks, vs, causal, scale, rows, o_ref, p, split)
    del p
    full = bound + 0.5 * ulp_bf16(np.abs(o_ref) * (1 + 2.0 ** -7)) + 1e-6
    err = np.abs(o_np - o_ref)
    ratio = float((err / full).max())
    ref_ss = float((o_ref ** 2).sum())
    rel_rms = float(np.sqrt((err ** 2).sum() / ref_ss)) if ref_ss > 0 else 0.0
    lrel = np.abs(lse_np - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    lse_worst = float(lrel.max())
    _say(f"    {name}: max_abs {float(err.max()):.3e} rel_rms {rel_rms:.3e} elem_ratio {ratio:.3f} "
         f"lse_rel {lse_worst:.3e}")
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()
    assert ratio <= 1.0, f"{name}: O element error {ratio:.3f} x its bound"
    assert rel_rms <= U8, f"{name}: O rel-RMS error {rel_rms:.3e} > 2^-4"
    assert lse_worst <= LSE_REL, f"{name}: lse relative error {lse_worst:.3e}"
    return rel_rms


@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(N, causal):
    _run(f"ragged N{N}", 2, 4, 2, N, causal, seed=3000 + N)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_key_split(causal):
    """One head of 2048 rows: too few blocks for the CUs, so the keys split
    and the combine kernel merges the BF16 partial outputs (FP32 lse values)."""
    _run("split 1x1x2048", 1, 1, 1, 2048, causal, seed=3101)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 1), (32, 1)])
def test_fp8_gqa(Hq, Hkv):
    _run(f"gqa {Hq}/{Hkv}", 1, Hq, Hkv, 384, True, seed=3200 + Hq * 10 + Hkv)


@pytest.mark.parametrize("scale,q_sign", [(0.0, 1.0), (-0.2, 1.0), (0.2, -1.0)])
def test_fp8_scale_edges(scale, q_sign):
    for causal in (False, True):
        _run(f"scale {scale} q_sign {q_sign}", 1, 2, 1, 300, causal, seed=3300, scale=scale, q_sign=q_sign)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_32_heads_4k(causal):
    """The 32-head N=4096 workload shape, 1,024 sampled rows per head (as the BF16 pass)."""
    _run("1x32x4096 d128", 1, 32, 32, 4096, causal, seed=3, sampled=1024)


@pytest.mark.parametrize("N", [1, 63, 100, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_d64_ragged(N, causal):
    _run(f"d64 ragged N{N}", 2, 4, 2, N, causal, seed=3400 + N, d=64)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_d64_key_split_gqa(causal):
    """d = 64 with grouped keys on one batch of 2 query heads: the keys split."""
    _run("d64 split 1x2x2048", 1, 2, 1, 2048, causal, seed=3501, d=64)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_d64_32_heads_4k(causal):
    _run("1x32x4096 d64", 1, 32, 32, 4096, causal, seed=4, sampled=1024, d=64)


def _quantize(x):
    """Per-tensor E4M3 codes of x (amax maps to 448) and the dequantisation factor."""
    descale = float(np.abs(x).max()) / si.FP8_E4M3_MAX
    return si.fp8_e4m3_round_bits(x / descale), descale


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_growing_scores_rescale(causal):
    """Scores that grow by about 10 (base 2) per 64-key tile: the FP8 pass's
    row max (slack 2) moves on every tile, so O and l are rescaled each step."""
    N, d = 640, 128
    q, k, v = si.growing_score_inputs(N, d, seed=1600)
    (q8, qs), (k8, ks), (v8, vs) = _quantize(q), _quantize(k), _quantize(v)
    _run(f"growing N{N}", 1, 2, 2, N, causal, seed=1600, d=d, codes=(q8, k8, v8, qs, ks, vs))
