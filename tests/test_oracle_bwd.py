"""Pins for the FP64 backward oracle (attention_bwd_ref).

The pages give no gradient formulas, so nothing here restates them. Each check
ties the oracle to something independent: central finite differences of the
forward oracle's loss, torch's FP64 CPU autograd through
scaled_dot_product_attention, closed forms, and an invariance. The last test
plants mistakes in a copy of the formulas and shows the pins catch them.
"""
import numpy as np
import pytest
import torch

from oracle import fa_oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, g, causal, scale):
    o, _ = fa_oracle.attention_ref(q, k, v, causal, scale)
    return float((o * g).sum())


def _finite_diff(q, k, v, g, causal, scale, h=1e-6):
    """Central differences of sum(O * G) with respect to every input element."""
    grads = []
    for x in (q, k, v):
        gx = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + h
            up = _loss(q, k, v, g, causal, scale)
            x[i] = old - h
            dn = _loss(q, k, v, g, causal, scale)
            x[i] = old
            gx[i] = (up - dn) / (2 * h)
        grads.append(gx)
    return grads


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_finite_differences(causal):
    rng = np.random.default_rng(31 + causal)
    q, k, v = _rand(rng, 1, 4, 5, 3), _rand(rng, 1, 2, 5, 3), _rand(rng, 1, 2, 5, 3)
    g = _rand(rng, 1, 4, 5, 3)
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, causal, 0.7)
    fq, fk, fv = _finite_diff(q, k, v, g, causal, 0.7)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.max(np.abs(a - b)) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd_fp64(causal):
    rng = np.random.default_rng(41 + causal)
    B, Hq, Hkv, N, d = 2, 6, 2, 37, 16
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    g = _rand(rng, B, Hq, N, d)
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    rep = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1), is_causal=causal, scale=scale)
    o.backward(torch.tensor(g))
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, causal, scale)
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd_fp64_across_row_chunks(causal):
    """N spans three of the oracle's row chunks (256 rows each, the last one
    ragged) with GQA: the dK/dV sums over chunks and over a group's query heads,
    and the dQ rows of every chunk, match torch's FP64 autograd. A second call
    on a seeded subset of rows and keys returns the same rows of those results."""
    rng = np.random.default_rng(43 + causal)
    B, Hq, Hkv, N, d = 1, 4, 2, 600, 8
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    g = _rand(rng, B, Hq, N, d)
    scale = 0.45
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    rep = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1), is_causal=causal, scale=scale)
    o.backward(torch.tensor(g))
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, causal, scale)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(mine - ref)) < 1e-11 * max(1.0, np.max(np.abs(ref)))
    rows = np.sort(rng.choice(N, 40, replace=False))
    keys = np.stack([np.sort(rng.choice(N, 30, replace=False)) for _ in range(Hkv)])
    dqs, dks, dvs = fa_oracle.attention_bwd_ref(q, k, v, g, causal, scale, rows=rows, key_rows=keys)
    assert np.max(np.abs(dqs - tq.grad.numpy()[:, :, rows])) < 1e-11
    for h in range(Hkv):
        assert np.max(np.abs(dks[:, h] - tk.grad.numpy()[:, h, keys[h]])) < 1e-11
        assert np.max(np.abs(dvs[:, h] - tv.grad.numpy()[:, h, keys[h]])) < 1e-11


def test_bwd_closed_forms():
    rng = np.random.default_rng(51)
    B, Hq, Hkv, N, d = 1, 2, 1, 9, 4
    q, k, g = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hq, N, d)
    # Every V row equal: O does not depend on P, so dQ = dK = 0; the columns of
    # P still sum each row's weight 1 into dV: sum_j dV_j = sum_i dO_i.
    v = np.repeat(_rand(rng, B, Hkv, 1, d), N, axis=2)
    for causal in (False, True):
        dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, causal, 0.9)
        assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
        assert np.max(np.abs(dv.sum(axis=2) - g.sum(axis=(1, 2))[:, None])) < 1e-12
    # Scale 0: uniform weights; dQ = dK = 0 and dV_j = (1/N) sum_i dO_i (non-causal),
    # sum over i >= j of dO_i / (i + 1) (causal).
    v = _rand(rng, B, Hkv, N, d)
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, False, 0.0)
    assert np.max(np.abs(dq)) == 0 and np.max(np.abs(dk)) == 0
    assert np.max(np.abs(dv[0, 0] - g[0].sum(axis=(0, 1)) / N)) < 1e-13
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, True, 0.0)
    w = 1.0 / np.arange(1, N + 1)
    want = np.stack([(g[0, :, j:] * w[j:, None]).sum(axis=(0, 1)) for j in range(N)])
    assert np.max(np.abs(dv[0, 0] - want)) < 1e-13


def test_bwd_permutation_invariance():
    """Permuting K and V rows together permutes dK, dV rows and keeps dQ (non-causal)."""
    rng = np.random.default_rng(61)
    q, k, v, g = _rand(rng, 1, 2, 11, 5), _rand(rng, 1, 2, 11, 5), _rand(rng, 1, 2, 11, 5), _rand(rng, 1, 2, 11, 5)
    perm = rng.permutation(11)
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, False, 0.4)
    dq2, dk2, dv2 = fa_oracle.attention_bwd_ref(q, k[:, :, perm], v[:, :, perm], g, False, 0.4)
    assert np.max(np.abs(dq - dq2)) < 1e-13
    assert np.max(np.abs(dk[:, :, perm] - dk2)) < 1e-13
    assert np.max(np.abs(dv[:, :, perm] - dv2)) < 1e-13


def test_bwd_row_selection():
    rng = np.random.default_rng(71)
    q, k, v, g = _rand(rng, 1, 2, 300, 4), _rand(rng, 1, 1, 300, 4), _rand(rng, 1, 1, 300, 4), _rand(rng, 1, 2, 300, 4)
    dq, dk, dv = fa_oracle.attention_bwd_ref(q, k, v, g, True, 0.5)
    rows, keys = np.array([0, 17, 255, 256, 299]), np.array([[3, 128, 299]])
    dqs, dks, dvs = fa_oracle.attention_bwd_ref(q, k, v, g, True, 0.5, rows=rows, key_rows=keys)
    assert np.max(np.abs(dqs - dq[:, :, rows])) < 1e-13
    assert np.max(np.abs(dks - dk[:, :, keys[0]])) < 1e-13
    assert np.max(np.abs(dvs - dv[:, :, keys[0]])) < 1e-13


def _pins_hold(bwd):
    """Finite differences on one tiny case, both masks, against a backward function."""
    rng = np.random.default_rng(81)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 4, 3)
    g = _rand(rng, 1, 2, 4, 3)
    ok = True
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, g, causal, 0.8)
        fq, fk, fv = _finite_diff(q, k, v, g, causal, 0.8)
        ok &= all(np.max(np.abs(a - b)) < 1e-6 for a, b in ((dq, fq), (dk, fk), (dv, fv)))
    return ok


def _mutant(kind):
    """The same chain rule with one planted mistake (one head, no GQA)."""
    def bwd(q, k, v, do, causal, scale):
        _, _, p = fa_oracle.attention_ref(q, k, v, causal, scale, return_p=True)
        p, qh, kh, vh, doh = p[0], q[0], np.repeat(k[0], 2, 0), np.repeat(v[0], 2, 0), do[0]
        dp = doh @ vh.transpose(0, 2, 1)
        dsum = (p * dp).sum(-1, keepdims=True)
        if kind == "minus_D_sign":
            dsum = -dsum
        ds = p * (dp - dsum) if kind != "no_P_in_dS" else (dp - dsum)
        dq = scale * ds @ kh
        dk = (ds.transpose(0, 2, 1) @ qh) * (1.0 if kind == "no_scale_dK" else scale)
        dv = p.transpose(0, 2, 1) @ doh if kind != "P_not_transposed" else p @ doh
        return dq[None], dk.sum(0)[None, None], dv.sum(0)[None, None]
    return bwd


def test_bwd_pins_catch_planted_mistakes():
    assert _pins_hold(fa_oracle.attention_bwd_ref)
    assert _pins_hold(_mutant("none"))
    for kind in ("minus_D_sign", "no_P_in_dS", "no_scale_dK", "P_not_transposed"):
        assert not _pins_hold(_mutant(kind)), kind
