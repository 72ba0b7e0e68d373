"""Shared helpers for the GPU parity tests (device upload and the error gates).

Tolerances:
  * official: O max abs error <= 1e-2; lse error |dlse| / max(|lse|, 1) <= 1e-3
    (the lse denominator is floored at 1 because causal early rows have lse near 0).
    The O max-abs gate is stated for the workloads, which all use scale 1/sqrt(d);
    tests at other scales (much sharper softmax, |O| up to ~4, where half a BF16
    ulp alone is 0.0078) are gated by the derived element bound below instead.
  * internal, element-wise, derived from the kernel's arithmetic. The kernel
    computes O_i = sum_j bf16(p_ij) v_j / l_i with p and l in FP32 and rounds O
    to BF16 once. With bf16(p) = p (1 + e), |e| <= 2^-8 (the unit roundoff of
    an 8-bit significand), the P rounding moves O_i by at most
    2^-8 sum_j p_ij |v_j| / l_i = 2^-8 (P|V|)_i, and the final rounding by half
    a BF16 unit in the last place. FP32 accumulation and the exp2/log2 units
    add relative errors near 1e-6. Hence
        |O_gpu - O_ref| <= 0.5 ulp_bf16(|O_ref| (1 + 2^-7))
                           + 1.125 * 2^-8 (P|V|)_ref + 1e-6,
    where (P|V|)_ref is the oracle's attention output with V replaced by |V|.
  * internal, aggregate: relative RMS error of O <= 2^-8.
  * key splits: when a call splits the keys, each split's normalised partial
    O_c is rounded to BF16 before the log-sum-exp combine, which moves O_i by
    at most 2^-8 sum_c w_c |O_c| / sum_c w_c <= 2^-8 (P|V|)_i (|O_c| <= the
    split's own P|V|, and the weights w_c recombine those into P|V|); the
    element bound then takes 2.125 * 2^-8 (P|V|) instead of 1.125.
"""
import numpy as np
import torch

O_MAX_ABS = 1e-2
LSE_REL = 1e-3
O_REL_RMS = 2.0 ** -8


def have_gpu() -> bool:
    return torch.cuda.is_available()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """BF16 bit pattern array (uint16) -> contiguous bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers at |x| (normal range; 8-bit significand)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def elem_bound(o_ref: np.ndarray, pabs_ref: np.ndarray, split: bool = False) -> np.ndarray:
    k = 2.125 if split else 1.125
    return 0.5 * ulp_bf16(np.abs(o_ref) * (1 + 2.0 ** -7)) + k * 2.0 ** -8 * pabs_ref + 1e-6


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, pabs_ref: np.ndarray, what: str,
            flat_gate: bool = True, split: bool = False) -> dict:
    err = np.abs(o_gpu - o_ref)
    finite = bool(np.isfinite(o_gpu).all())
    max_abs = float(err.max()) if err.size else 0.0
    rel_rms = float(np.sqrt((err ** 2).sum() / max((o_ref ** 2).sum(), 1e-300))) if err.size else 0.0
    worst = float((err / elem_bound(o_ref, pabs_ref, split)).max()) if err.size else 0.0
    stats = {"max_abs": max_abs, "rel_rms": rel_rms, "elem_ratio": worst}
    print(f"    {what}: {stats}", flush=True)
    assert finite, f"{what}: non-finite O"
    if flat_gate:
        assert max_abs <= O_MAX_ABS, f"{what}: O max abs error {max_abs:.3e} > {O_MAX_ABS}"
    assert rel_rms <= O_REL_RMS, f"{what}: O rel-RMS error {rel_rms:.3e} > {O_REL_RMS:.3e}"
    assert worst <= 1.0, f"{what}: O element error {worst:.3f} x the derived element bound"
    return stats


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str) -> float:
    rel = np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    worst = float(rel.max()) if rel.size else 0.0
    print(f"    {what}: lse rel {worst:.3e}", flush=True)
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite lse"
    assert worst <= LSE_REL, f"{what}: lse relative error {worst:.3e} > {LSE_REL}"
    return worst


U_BF16 = 2.0 ** -8  # unit roundoff of an 8-bit significand


def bwd_elem_bounds(q, k, v, do, causal, scale):
    """Element-wise error bounds for the GPU backward pass (FP64 inputs; small sizes).

    The kernels recompute P = 2^(S c - lse2) in FP32, round P and dS to BF16 for
    the products dV = P^T dO and dK = dS^T Q (and dS for dQ = dS K), and take
    delta_i = sum_t dO_it O_it from the forward's BF16 output O. With u = 2^-8:
      * |O_gpu - O| <= 0.5 ulp(|O| (1 + 2^-7)) + 1.125 u (P|V|)   (the forward's bound),
        so |delta_gpu - delta|_i <= E_i = sum_t |dO_it| (that bound)_it;
      * dV: |err| <= 1.01 u (P^T |dO|) + 0.5 ulp + FP32 terms;
      * dK: |err| <= |scale| ((P * E + u |dS|)^T |Q|) + 0.5 ulp + FP32 terms;
      * dQ: |err| <= |scale| ((P * E + u |dS|) |K|) + 0.5 ulp + FP32 terms;
    the FP32 terms (accumulation, exp2 and lse) take 1e-5 of the same sums with
    |dP| + |delta| in place of the BF16 terms. The 0.5 ulp of the output's final
    rounding is added by the caller (it needs the reference value).
    Returns the bounds for dq [B,Hq,N,d], dk and dv [B,Hkv,N,d], without the ulp term.
    """
    from oracle import fa_oracle
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    bq = np.zeros((B, Hq, N, d))
    bk = np.zeros((B, Hkv, N, d))
    bv = np.zeros((B, Hkv, N, d))
    u = U_BF16
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qh, kh, vh, doh = q[b, h], k[b, g], v[b, g], do[b, h]
            o, _, p = fa_oracle.attention_ref(qh[None, None], kh[None, None], vh[None, None], causal, scale,
                                              return_p=True)
            o, p = o[0, 0], p[0, 0]
            pv_abs = p @ np.abs(vh)
            e = (np.abs(doh) * (0.5 * ulp_bf16(np.abs(o) * (1 + 2.0 ** -7)) + 1.125 * u * pv_abs)).sum(1)
            dp = doh @ vh.T
            dlt = (p * dp).sum(1)
            ds = p * (dp - dlt[:, None])
            w_q = p * e[:, None] + u * np.abs(ds) + 1e-5 * p * (np.abs(dp) + np.abs(dlt)[:, None])
            bq[b, h] = abs(scale) * (w_q @ np.abs(kh))
            bk[b, g] += abs(scale) * (w_q.T @ np.abs(qh))
            bv[b, g] += (1.01 * u + 1e-5) * (p.T @ np.abs(doh))
    return bq, bk, bv


def check_grad(name, got, ref, bound, what):
    """got/ref/bound FP64 arrays of one gradient; bound excludes the final rounding."""
    err = np.abs(got - ref)
    full = bound + 0.5 * ulp_bf16(np.abs(ref) * (1 + 2.0 ** -7)) + 1e-6
    ratio = float((err / full).max()) if err.size else 0.0
    ref_ss = float((ref ** 2).sum())
    # (a gradient that is exactly zero, e.g. dQ and dK of a single key, has no relative error)
    rel = f"{float(np.sqrt((err ** 2).sum() / ref_ss)):.3e}" if ref_ss > 0 else "n/a (zero reference)"
    print(f"    {what} {name}: max_abs {float(err.max()) if err.size else 0.0:.3e} rel_rms {rel} "
          f"elem_ratio {ratio:.3f}", flush=True)
    assert np.isfinite(got).all(), f"{what} {name}: non-finite values"
    assert ratio <= 1.0, f"{what} {name}: element error {ratio:.3f} x its bound"
    return ratio
