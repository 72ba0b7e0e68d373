"""Pins for the FP64 oracle: values the pages print and facts the definition fixes.

Nothing here compares the oracle with itself. Each check ties it to something
independent: the printed toy run, pure-Python brute force, closed forms,
invariants, or torch's FP64 CPU scaled_dot_product_attention. The last test
plants mistakes in a copy of the oracle and shows that the pins catch them.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import fa_oracle
from oracle import fa_online
from seeded_inputs import bf16_bits_to_f32, bf16_round_bits, sample_rows


def _read_golden(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ toy run

def test_toy_run_printed_values(golden_dir):
    """Printed toy run ("A toy run, and the traffic it saves"): m, l and weights."""
    g = _read_golden(os.path.join(golden_dir, "toy_online_softmax.txt"))
    scores = [float(x) for x in g["scores"]]
    weights = [float(x) for x in g["weights"]]
    wdec = int(g["weights_decimals"][0])
    sdec = int(g["sum_decimals"][0])
    # One query, d = 1, scale = 1: q.k_j = k_j, so S equals the printed scores.
    q = np.ones((1, 1, 1, 1))
    k = np.array(scores).reshape(1, 1, 4, 1)
    v = np.eye(4).reshape(1, 1, 4, 4)  # one-hot V rows: O recovers the weights
    o, lse, p = fa_oracle.attention_ref(q, k, v, causal=False, scale=1.0, return_p=True)
    assert np.round(o[0, 0, 0], wdec).tolist() == weights
    assert np.round(p[0, 0, 0], wdec).tolist() == weights
    m_final = max(scores)
    assert m_final == float(g["max_final"][0])
    l_final = math.exp(lse[0, 0, 0] - m_final)  # running sum relative to the final max
    assert round(l_final, sdec) == float(g["sum_final"][0])
    # Closed form: l = 1 + e^-1 + e^-2 + e^-3 (scores 3, 2, 1, 0 against max 3).
    assert abs(l_final - (1 + math.exp(-1) + math.exp(-2) + math.exp(-3))) < 1e-15


@pytest.mark.parametrize("blocks", [(2, 2), (3, 1), (1, 3)])
def test_toy_run_online_two_blocks(golden_dir, blocks):
    """The streaming update reproduces the printed run for every two-block split."""
    g = _read_golden(os.path.join(golden_dir, "toy_online_softmax.txt"))
    scores = [float(x) for x in g["scores"]]
    trace = fa_online.running_stats(scores, list(blocks))
    assert trace[-1][0] == float(g["max_final"][0])
    assert round(trace[-1][1], int(g["sum_decimals"][0])) == float(g["sum_final"][0])
    if blocks == (2, 2):
        assert trace[0][0] == float(g["max_after_block1"][0])
    # The tiled model's weights also match the printed ones.
    q = np.ones((1, 1))
    k = np.array(scores).reshape(4, 1)
    o, lse = fa_online.tiled_attention(q, k, np.eye(4), scale=1.0, block_q=1, block_kv=blocks[0])
    assert np.round(o[0], 4).tolist() == [float(x) for x in g["weights"]]


# ------------------------------------------------------------ brute force

def _brute(q, k, v, causal, scale):
    """Pure-Python triple loop with math.fsum; q [Hq][N][d], k/v [Hkv][N_k][d]."""
    Hq, N, d = len(q), len(q[0]), len(q[0][0])
    n_keys = len(k[0])
    group = Hq // len(k)
    o = [[[0.0] * d for _ in range(N)] for _ in range(Hq)]
    lse = [[0.0] * N for _ in range(Hq)]
    for h in range(Hq):
        kh, vh = k[h // group], v[h // group]
        for i in range(N):
            js = [j for j in range(n_keys) if (not causal or j <= i)]
            s = [scale * math.fsum(q[h][i][t] * kh[j][t] for t in range(d)) for j in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            for t in range(d):
                o[h][i][t] = math.fsum(w[a] * vh[j][t] for a, j in enumerate(js)) / l
            lse[h][i] = m + math.log(l)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("N,d,Hq,Hkv,causal", [(1, 4, 1, 1, False), (5, 3, 2, 1, False),
                                               (7, 4, 4, 2, True), (8, 5, 2, 2, True),
                                               (6, 2, 3, 3, False)])
def test_brute_force_tiny(N, d, Hq, Hkv, causal):
    rng = np.random.default_rng(100 + N * 10 + d)
    q, k, v = _rand(rng, 1, Hq, N, d), _rand(rng, 1, Hkv, N, d), _rand(rng, 1, Hkv, N, d)
    scale = 0.7
    o, lse = fa_oracle.attention_ref(q, k, v, causal, scale)
    ob, lseb = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), causal, scale)
    assert np.max(np.abs(o[0] - ob)) < 1e-13
    assert np.max(np.abs(lse[0] - lseb)) < 1e-13


# ------------------------------------------------------------ closed forms

def test_single_key_closed_form():
    """N = 1: the only weight is 1, so O = V_0 and lse = scale q.k_0."""
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 1, 16), _rand(rng, 1, 2, 1, 16), _rand(rng, 1, 2, 1, 16)
    for causal in (False, True):
        o, lse = fa_oracle.attention_ref(q, k, v, causal, 0.25)
        assert np.allclose(o, v, rtol=0, atol=1e-15)
        assert np.allclose(lse[..., 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)


def test_value_probes_and_row_sums():
    """V = ones gives O = 1; V = identity recovers P, whose rows sum to 1."""
    rng = np.random.default_rng(4)
    N = 12
    q, k = _rand(rng, 1, 1, N, 8), _rand(rng, 1, 1, N, 8)
    for causal in (False, True):
        o, _ = fa_oracle.attention_ref(q, k, np.ones((1, 1, N, 8)), causal, 0.5)
        assert np.max(np.abs(o - 1.0)) < 1e-14
        o, _, p = fa_oracle.attention_ref(q, k, np.eye(N).reshape(1, 1, N, N), causal, 0.5, return_p=True)
        assert np.max(np.abs(o - p)) < 1e-15
        assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-15
        assert (p >= 0).all()
        if causal:
            assert np.all(np.triu(p[0, 0], 1) == 0.0)


def test_equal_scores_give_mean():
    """Equal scores: O is the mean of the visible V rows and lse = s + ln(count)."""
    rng = np.random.default_rng(5)
    N, d = 20, 6
    q = _rand(rng, 1, 1, N, d)
    krow = _rand(rng, d)
    k = np.broadcast_to(krow, (1, 1, N, d)).copy()
    v = _rand(rng, 1, 1, N, d)
    scale = 0.3
    s = scale * q[0, 0] @ krow
    o, lse = fa_oracle.attention_ref(q, k, v, False, scale)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(0))) < 1e-14
    assert np.max(np.abs(lse[0, 0] - (s + math.log(N)))) < 1e-13
    o, lse = fa_oracle.attention_ref(q, k, v, True, scale)
    prefix_mean = np.cumsum(v[0, 0], 0) / np.arange(1, N + 1)[:, None]
    assert np.max(np.abs(o[0, 0] - prefix_mean)) < 1e-14
    assert np.max(np.abs(lse[0, 0] - (s + np.log(np.arange(1, N + 1))))) < 1e-13


def test_zero_scale():
    """scale = 0: every score is 0, lse = ln N (causal ln(i+1)), O = mean of V."""
    rng = np.random.default_rng(6)
    N = 9
    q, k, v = _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 4), _rand(rng, 1, 1, N, 4)
    o, lse = fa_oracle.attention_ref(q, k, v, False, 0.0)
    assert np.max(np.abs(lse - math.log(N))) < 1e-15
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(0))) < 1e-15
    o, lse = fa_oracle.attention_ref(q, k, v, True, 0.0)
    assert np.max(np.abs(lse[0, 0] - np.log(np.arange(1, N + 1)))) < 1e-15


def test_joint_kv_permutation_invariance():
    """Permuting K and V rows together leaves non-causal O and lse unchanged."""
    rng = np.random.default_rng(7)
    N = 64
    q, k, v = _rand(rng, 1, 2, N, 16), _rand(rng, 1, 2, N, 16), _rand(rng, 1, 2, N, 16)
    perm = rng.permutation(N)
    o1, l1 = fa_oracle.attention_ref(q, k, v, False, 0.25)
    o2, l2 = fa_oracle.attention_ref(q, k[:, :, perm], v[:, :, perm], False, 0.25)
    assert np.max(np.abs(o1 - o2)) < 1e-13
    assert np.max(np.abs(l1 - l2)) < 1e-13
    # A K-only permutation is a different problem: the check has teeth.
    o3, _ = fa_oracle.attention_ref(q, k[:, :, perm], v, False, 0.25)
    assert np.max(np.abs(o1 - o3)) > 1e-3


# ---------------------------------------------------------- library routine

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    """torch's FP64 CPU scaled_dot_product_attention is an independent textbook routine."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, N, d = 2, 4, 2, 37, 16
    q, k, v = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa_oracle.attention_ref(q, k, v, causal, scale)
    group = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k, group, axis=1))
    vt = torch.from_numpy(np.repeat(v, group, axis=1))
    qt = torch.from_numpy(q)
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    assert np.max(np.abs(o - ot.numpy())) < 1e-13
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) < 1e-13


# ------------------------------------------------------------ tiled algebra

@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_online_tiled_equals_definition_p2_harness(block):
    """The harness shape of "The Tiling Algorithm": seq 1024, d 64, seed 0."""
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1024, 64)) for _ in range(3))
    o_t, lse_t = fa_online.tiled_attention(q, k, v, 1 / 8.0, block, block)
    o, lse = fa_oracle.attention_ref(q[None, None], k[None, None], v[None, None], False, 1 / 8.0)
    assert np.max(np.abs(o_t - o[0, 0])) < 1e-12
    assert np.max(np.abs(lse_t - lse[0, 0])) < 1e-12


@pytest.mark.parametrize("N,bq,bk", [(1000, 64, 128), (129, 128, 64), (100, 32, 48)])
def test_online_tiled_causal_ragged(N, bq, bk):
    rng = np.random.default_rng(N)
    q, k, v = (rng.standard_normal((N, 32)) for _ in range(3))
    o_t, lse_t = fa_online.tiled_attention(q, k, v, 0.2, bq, bk, causal=True)
    o, lse = fa_oracle.attention_ref(q[None, None], k[None, None], v[None, None], True, 0.2)
    assert np.max(np.abs(o_t - o[0, 0])) < 1e-12
    assert np.max(np.abs(lse_t - lse[0, 0])) < 1e-12


# ------------------------------------------------------------ split-KV decode

@pytest.mark.parametrize("L,splits", [(8192, 16), (1000, 16), (5, 4), (7, 7), (33, 1)])
def test_split_combine_equals_one_pass(L, splits):
    rng = np.random.default_rng(L + splits)
    B, Hq, Hkv, d = 2, 8, 2, 16
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    o, lse = fa_oracle.decode_ref(q, k, v, 0.25)
    op, lp = fa_oracle.split_decode_partials_ref(q, k, v, 0.25, splits)
    oc, lc = fa_oracle.combine_ref(op, lp)
    assert np.max(np.abs(o - oc)) < 1e-12
    assert np.max(np.abs(lse - lc)) < 1e-12
    if L == 5:  # chunk = 2 keys: the fourth chunk is empty
        assert np.isneginf(lp[..., 3]).all()


def test_decode_is_last_causal_row():
    """One decode query equals the last row of causal attention on the same keys."""
    rng = np.random.default_rng(11)
    N, d = 50, 8
    q, k, v = _rand(rng, 1, 4, N, d), _rand(rng, 1, 2, N, d), _rand(rng, 1, 2, N, d)
    o, lse = fa_oracle.attention_ref(q, k, v, True, 0.35)
    od, lsed = fa_oracle.decode_ref(q[:, :, N - 1], k, v, 0.35)
    assert np.max(np.abs(od - o[:, :, N - 1])) < 1e-14
    assert np.max(np.abs(lsed - lse[:, :, N - 1])) < 1e-14


def test_decode_varlen_is_causal_row_at_its_length():
    """Sequence b with len_b keys equals row len_b - 1 of causal attention over its
    padded cache: the causal mask, not slicing, limits the keys there. Padding
    holding NaN and huge values takes no part."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, L, d = 4, 4, 2, 40, 8
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    lens = np.array([1, 17, 39, 40])
    kp, vp = k.copy(), v.copy()
    for b, n in enumerate(lens):
        kp[b, :, n:] = np.nan
        vp[b, :, n:] = 1e30
    od, ld = fa_oracle.decode_varlen_ref(q, kp, vp, lens, 0.3)
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    for b, n in enumerate(lens):
        qc = np.repeat(q[b:b + 1], L, axis=2)  # the query at every row; row n - 1 is the one that counts
        o, lse = fa_oracle.attention_ref(qc, k[b:b + 1], v[b:b + 1], True, 0.3, rows=np.full((Hq, 1), n - 1))
        assert np.max(np.abs(od[b] - o[0, :, 0])) < 1e-14
        assert np.max(np.abs(ld[b] - lse[0, :, 0])) < 1e-14


def test_decode_varlen_closed_forms():
    rng = np.random.default_rng(15)
    B, Hq, Hkv, L, d = 4, 4, 2, 9, 8
    q, k, v = _rand(rng, B, Hq, 1, d), _rand(rng, B, Hkv, L, d), _rand(rng, B, Hkv, L, d)
    od, ld = fa_oracle.decode_varlen_ref(q, k, v, [1, 0, -3, 99], 0.5)
    for h in range(Hq):  # one key: O = v_0, lse = scale q.k_0
        assert np.allclose(od[0, h], v[0, h // 2, 0], atol=0, rtol=1e-15)
        assert math.isclose(ld[0, h], 0.5 * float(np.dot(q[0, h, 0], k[0, h // 2, 0])), rel_tol=1e-14)
    assert (od[1:3] == 0).all() and np.isneginf(ld[1:3]).all()  # no key (a negative count means none)
    of, lf = fa_oracle.decode_ref(q[3:], k[3:], v[3:], 0.5)  # a count past L means all L keys
    assert np.max(np.abs(od[3] - of[0])) < 1e-15 and np.max(np.abs(ld[3] - lf[0])) < 1e-15


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(12)
    N = 300
    q, k, v = _rand(rng, 1, 2, N, 8), _rand(rng, 1, 2, N, 8), _rand(rng, 1, 2, N, 8)
    rows = np.stack([sample_rows(9, h, N, 40) for h in range(2)])
    for causal in (False, True):
        o, lse = fa_oracle.attention_ref(q, k, v, causal, 0.3)
        os_, ls_ = fa_oracle.attention_ref(q, k, v, causal, 0.3, rows=rows)
        for h in range(2):
            # Same rows, different BLAS blocking: equal up to FP64 reassociation.
            assert np.max(np.abs(os_[0, h] - o[0, h, rows[h]])) < 1e-14
            assert np.max(np.abs(ls_[0, h] - lse[0, h, rows[h]])) < 1e-14


def test_bf16_rounding_helpers():
    """RNE to BF16: ties go to even; the widened values are exact BF16 numbers."""
    x = np.array([1.0 + 1 / 256, 1.0 + 3 / 256, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = bf16_round_bits(x)
    assert bits.tolist()[:3] == [0x3F80, 0x3F82, 0xC020]
    w = bf16_bits_to_f32(bits)
    assert np.array_equal(bf16_round_bits(w), bits)
    rng = np.random.default_rng(1)
    y = rng.standard_normal(10000).astype(np.float32)
    yb = bf16_bits_to_f32(bf16_round_bits(y))
    assert np.max(np.abs(yb - y) / np.abs(y)) <= 2.0 ** -8  # unit roundoff, 8-bit significand


# ---------------------------------------------------------- planted mistakes

def _pins_hold(mod):
    """A compact set of the pins above, run against a (possibly mutated) oracle.

    An oracle that raises on a pin's input fails that pin.
    """
    try:
        return _pins_hold_inner(mod)
    except ValueError:
        return False


def _pins_hold_inner(mod):
    rng = np.random.default_rng(21)
    ok = True
    # brute force with GQA and causal
    q, k, v = _rand(rng, 1, 4, 6, 3), _rand(rng, 1, 2, 6, 3), _rand(rng, 1, 2, 6, 3)
    for causal in (False, True):
        o, lse = mod.attention_ref(q, k, v, causal, 0.6)
        ob, lb = _brute(q[0].tolist(), k[0].tolist(), v[0].tolist(), causal, 0.6)
        ok &= bool(np.max(np.abs(o[0] - ob)) < 1e-12 and np.max(np.abs(lse[0] - lb)) < 1e-12)
    # toy run
    o, lse = mod.attention_ref(np.ones((1, 1, 1, 1)), np.array([2.0, 1, 0, 3]).reshape(1, 1, 4, 1),
                               np.eye(4).reshape(1, 1, 4, 4), False, 1.0)
    ok &= np.round(o[0, 0, 0], 4).tolist() == [0.2369, 0.0871, 0.0321, 0.6439]
    # decode vs combine
    qd, kd, vd = _rand(rng, 1, 2, 1, 4), _rand(rng, 1, 1, 20, 4), _rand(rng, 1, 1, 20, 4)
    od, ld = mod.decode_ref(qd, kd, vd, 0.5)
    oc, lc = mod.combine_ref(*mod.split_decode_partials_ref(qd, kd, vd, 0.5, 3))
    ok &= bool(np.max(np.abs(od - oc)) < 1e-12 and np.max(np.abs(ld - lc)) < 1e-12)
    ob, lb = _brute(qd[0].tolist(), kd[0].tolist(), vd[0].tolist(), False, 0.5)
    ok &= bool(np.max(np.abs(od[0] - ob[:, 0])) < 1e-12)
    # variable-length decode: brute force over the first n keys
    for n in (1, 7, 20):
        ov, lv = mod.decode_varlen_ref(qd, kd, vd, [n], 0.5)
        ob, lb = _brute(qd[0].tolist(), kd[0, :, :n].tolist(), vd[0, :, :n].tolist(), False, 0.5)
        ok &= bool(np.max(np.abs(ov[0] - ob[:, 0])) < 1e-12 and np.max(np.abs(lv[0] - lb[:, 0])) < 1e-12)
    return ok


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _pins_hold(fa_oracle)
    orig = fa_oracle._standard_attention_rows

    def no_scale(qr, k, v, scale, ids, causal):
        return orig(qr, k, v, 1.0, ids, causal)

    def mask_diag(qr, k, v, scale, ids, causal):  # hides j == i as well
        if not causal:
            return orig(qr, k, v, scale, ids, causal)
        s = scale * (qr @ k.T)
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols < ids[:, None], s, -np.inf)
        s[~np.isfinite(s).any(axis=1), 0] = 0.0
        m = s.max(1)
        p = np.exp(s - m[:, None])
        l = p.sum(1)
        return (p / l[:, None]) @ v, m + np.log(l), p / l[:, None]

    def no_normalise(qr, k, v, scale, ids, causal):
        o, lse, p = orig(qr, k, v, scale, ids, causal)
        return o * np.exp(lse - (scale * (qr @ k.T)).max(1))[:, None], lse, p

    def lse_without_max(qr, k, v, scale, ids, causal):
        o, lse, p = orig(qr, k, v, scale, ids, causal)
        s = scale * (qr @ k.T)
        return o, lse - s.max(1), p

    def transposed_kv_roles(qr, k, v, scale, ids, causal):
        return orig(qr, v, k, scale, ids, causal)

    for bad in (no_scale, mask_diag, no_normalise, lse_without_max, transposed_kv_roles):
        monkeypatch.setattr(fa_oracle, "_standard_attention_rows", bad)
        assert not _pins_hold(fa_oracle), bad.__name__
        monkeypatch.setattr(fa_oracle, "_standard_attention_rows", orig)

    # A wrong combine weight and a wrong GQA mapping are caught too.
    orig_combine = fa_oracle.combine_ref
    monkeypatch.setattr(fa_oracle, "combine_ref",
                        lambda o, l: (np.asarray(o).mean(-2), np.asarray(l).max(-1)))
    assert not _pins_hold(fa_oracle)
    monkeypatch.setattr(fa_oracle, "combine_ref", orig_combine)

    orig_attn = fa_oracle.attention_ref

    def wrong_group(q, k, v, causal, scale, rows=None, return_p=False):
        k2 = np.asarray(k)[:, np.arange(np.asarray(q).shape[1]) % np.asarray(k).shape[1]]
        v2 = np.asarray(v)[:, np.arange(np.asarray(q).shape[1]) % np.asarray(v).shape[1]]
        return orig_attn(q, k2, v2, causal, scale, rows, return_p)

    monkeypatch.setattr(fa_oracle, "attention_ref", wrong_group)
    assert not _pins_hold(fa_oracle)
    monkeypatch.setattr(fa_oracle, "attention_ref", orig_attn)

    # A variable-length decode that takes one key too many, or ignores the lengths.
    orig_varlen = fa_oracle.decode_varlen_ref
    for bad_lens in (lambda lens: [n + 1 for n in lens], lambda lens: [10 ** 9 for _ in lens]):
        monkeypatch.setattr(fa_oracle, "decode_varlen_ref",
                            lambda q, k, v, lens, scale, f=bad_lens: orig_varlen(q, k, v, f(lens), scale))
        assert not _pins_hold(fa_oracle)
    monkeypatch.setattr(fa_oracle, "decode_varlen_ref", orig_varlen)
