"""GPU parity of the backward pass against the FP64 oracle, through the C ABI.

The GPU runs its own forward (o, lse), then the backward from those and a
seeded upstream gradient; the oracle differentiates the exact attention of the
same BF16-valued inputs. Small cases are gated element-wise by a bound derived
from the kernels' arithmetic (gpu_helpers.bwd_elem_bounds); the 32-head 4K
workload is checked on eight heads' sampled rows and keys by the same bound, and
on every head by an identity of the exact gradients (the dV column sums).
"""
import sys

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import bwd_elem_bounds, check_grad, have_gpu, to_dev, to_f64
from oracle import fa_oracle

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _gpu_bwd(qb, kb, vb, gb, causal, scale):
    import torch
    import exact_tiled_attention_fa_amd as fa
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_f64(dq), to_f64(dk), to_f64(dv)


def _inputs(B, Hq, Hkv, N, seed, d=128):
    case = si.FwdCase(f"bwd {B}x{Hq}/{Hkv}x{N}", B, Hq, Hkv, N, d, False, seed)
    qb, kb, vb = si.fwd_inputs(case)
    gb = si.normal_bf16(np.random.default_rng(seed + 10_000), (B, Hq, N, d))
    return qb, kb, vb, gb


def _run_small(B, Hq, Hkv, N, causal, seed, scale=None, d=128):
    scale = d ** -0.5 if scale is None else scale
    what = f"bwd B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal} scale={scale:.4g}"
    print(f"[bwd] {what} seed={seed}", flush=True)
    sys.stdout.flush()
    qb, kb, vb, gb = _inputs(B, Hq, Hkv, N, seed, d)
    dq, dk, dv = _gpu_bwd(qb, kb, vb, gb, causal, scale)
    qf, kf, vf, gf = (si.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb, gb))
    rq, rk, rv = fa_oracle.attention_bwd_ref(qf, kf, vf, gf, causal, scale)
    bq, bk, bv = bwd_elem_bounds(qf, kf, vf, gf, causal, scale)
    for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        check_grad(name, got, ref, bnd, what)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 2, 2, 256), (2, 4, 2, 200), (1, 1, 1, 1), (1, 3, 1, 67),
                                        (1, 2, 1, 1000), (1, 1, 1, 64)])
def test_bwd_small(B, Hq, Hkv, N, causal):
    _run_small(B, Hq, Hkv, N, causal, seed=700 + N + Hq)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(2, 16, 8, 300), (1, 24, 24, 130)])
def test_bwd_causal_head_groups(B, Hq, Hkv, N):
    """Causal grids interleave the blocks of one XCD's share of heads: here
    2 KV heads and 4 query heads per group, then 3 and 3."""
    _run_small(B, Hq, Hkv, N, True, seed=1400 + N + Hq)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_multi_query(causal, d):
    """16 query heads over one KV head: each key block's dK and dV sum over all 16 heads' tiles in
    one sweep."""
    _run_small(1, 16, 1, 200, causal, seed=1450 + d + int(causal), d=d)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.3])
def test_bwd_scale_edge_cases(scale):
    _run_small(1, 2, 1, 300, True, seed=800, scale=scale)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 2, 2, 256), (2, 4, 2, 200), (1, 1, 1, 1), (1, 3, 1, 67),
                                        (1, 2, 1, 1000)])
def test_bwd_small_d64(B, Hq, Hkv, N, causal):
    _run_small(B, Hq, Hkv, N, causal, seed=900 + N + Hq, d=64)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_bwd_scale_edge_cases_d64(scale):
    _run_small(1, 2, 1, 300, True, seed=950, scale=scale, d=64)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_32_heads_4k_sampled(causal):
    """The 32-head 4K shape (the bench's backward workload), all heads on the GPU.
    Eight heads, at least one in each XCD's range of the grid (four heads per
    XCD without causal masking; causal grids interleave the heads of a range),
    are compared on 1,024 seeded rows (dQ) and keys (dK, dV) with the derived
    element-wise bounds of the small cases."""
    B, Hq, N = 1, 32, 4096
    qb, kb, vb, gb = _inputs(B, Hq, Hq, N, seed=3)
    scale = 128 ** -0.5
    heads = [0, 5, 10, 15, 17, 22, 27, 31]
    print(f"[bwd] 1x32x4096 causal={causal} (heads {heads} sampled)", flush=True)
    dq, dk, dv = _gpu_bwd(qb, kb, vb, gb, causal, scale)
    sel = lambda x: si.bf16_bits_to_f32(x[:, heads]).astype(np.float64)
    qf, kf, vf, gf = sel(qb), sel(kb), sel(vb), sel(gb)
    rows = np.stack([si.sample_rows(3, h, N, 1024) for h in heads])
    rq, rk, rv = fa_oracle.attention_bwd_ref(qf, kf, vf, gf, causal, scale, rows=rows, key_rows=rows)
    bq, bk, bv = bwd_elem_bounds(qf, kf, vf, gf, causal, scale)
    pick = lambda x: np.stack([x[:, n, rows[n]] for n in range(len(heads))], axis=1)
    for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        got = np.stack([got[:, h, rows[n]] for n, h in enumerate(heads)], axis=1)
        check_grad(name, got, ref, pick(bnd), f"1x32x4096 causal={causal}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [(1, 32, 32, 4096, 128, False), (1, 32, 32, 4096, 128, True),
                                                 (1, 32, 8, 4096, 128, True), (2, 8, 2, 3000, 64, False)],
                         ids=["32x4k", "32x4k-causal", "gqa-causal", "d64-ragged"])
def test_bwd_dv_column_sums_every_head(B, Hq, Hkv, N, d, causal):
    """Every head at full size, by an identity of the exact gradients: each row of P sums to 1 over its
    visible keys, so the keys' dV = P^T dO add up to the query rows' dO, sum_j dV_j = sum_i dO_i (per KV
    head and column, summed over the heads of its group). The kernel's P is rounded to BF16 before the
    product (relative error <= 2^-8, so at most 2^-8 sum_i |dO_i| over all keys) and dV is stored in BF16
    (at most 2^-8 |dV_j| each); 2^-12 sum_i |dO_i| more covers the FP32 recomputation of P and the FP32
    sums. The bound is a worst case that grows with N, so this catches errors of whole heads or groups
    (mapping, grouping, scale, normalisation) on every head; single tiles are the sampled test's job."""
    import torch
    import exact_tiled_attention_fa_amd as fa
    what = f"B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}"
    print(f"[bwd] dV column sums {what}", flush=True)
    qb, kb, vb, gb = _inputs(B, Hq, Hkv, N, seed=41, d=d)
    q, k, v, g = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    o, lse = fa.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, g, causal=causal)
    torch.cuda.synchronize()
    G = Hq // Hkv
    dv64 = dv.double()
    g64 = g.double().reshape(B, Hkv, G, N, d)
    lhs = dv64.sum(dim=2)                                   # [B, Hkv, d]
    rhs = g64.sum(dim=(2, 3))
    bound = 2.0 ** -8 * dv64.abs().sum(dim=2) + (2.0 ** -8 + 2.0 ** -12) * g64.abs().sum(dim=(2, 3))
    err = (lhs - rhs).abs()
    ratio = float((err / bound).max())
    print(f"    {what}: max |sum dV - sum dO| / bound = {ratio:.3f}", flush=True)
    assert torch.isfinite(dv64).all() and ratio <= 1.0, f"{what}: dV column sums off by {ratio:.3f} x the bound"
