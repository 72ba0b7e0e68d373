"""Pins for the FP8 pieces: the oracle's E4M3 decoding, the FP8 attention
reference, and the seeded E4M3 encoder that prepares GPU inputs.

Each check ties a function to something it does not compute itself: the
format's closed-form values, torch's own float8_e4m3fn conversions, a brute
force nearest-code search, invariances and closed forms of attention, and
torch's FP64 CPU scaled_dot_product_attention. The last test plants mistakes
in copies of the decoder and shows the pins catch them.
"""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import fa_oracle

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _decode_pins_hold(decode) -> bool:
    v = decode(ALL)
    checks = [
        v[0x00] == 0.0 and not np.signbit(v[0x00]),
        v[0x80] == 0.0 and np.signbit(v[0x80]),
        v[0x01] == 2.0 ** -9,              # smallest subnormal
        v[0x07] == 7 * 2.0 ** -9,          # largest subnormal
        v[0x08] == 2.0 ** -6,              # smallest normal
        v[0x38] == 1.0,
        v[0x3C] == 1.5,
        v[0x7E] == 448.0,                  # largest finite
        np.isnan(v[0x7F]) and np.isnan(v[0xFF]),
        int(np.isnan(v).sum()) == 2,
    ]
    fin = v[:0x7F]
    checks.append(bool(np.all(np.diff(fin) > 0)))                        # increasing
    checks.append(bool(np.array_equal(v[0x80:0xFF], -v[:0x7F])))         # sign symmetry
    return all(bool(c) for c in checks)


def test_decode_closed_forms():
    assert _decode_pins_hold(fa_oracle.fp8_e4m3_value)


def test_decode_matches_torch():
    mine = fa_oracle.fp8_e4m3_value(ALL)
    ref = _torch_decode(ALL)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(ref[fin]))


def test_encoder_is_nearest_even():
    """seeded_inputs.fp8_e4m3_round_bits against a brute-force nearest search."""
    table = fa_oracle.fp8_e4m3_value(ALL)
    finite = np.where(np.isfinite(table))[0]
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.6, 4000),
        table[finite],
        (table[1:0x7E] + table[2:0x7F]) / 2,   # every positive tie
        -(table[1:0x7E] + table[2:0x7F]) / 2,
    ])
    codes = si.fp8_e4m3_round_bits(x)
    got = table[codes]
    for xi, gi, ci in zip(x, got, codes):
        d = np.abs(table[finite] - xi)
        best = finite[d == d.min()]
        if len(best) > 1:  # tie: the even code (and the sign of x for a zero)
            best = [b for b in best if b % 2 == 0]
        assert ci in best or (gi == 0 and table[best[0]] == 0), (xi, ci, best)


def test_encoder_matches_torch_in_range():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(5000) * 10.0 ** rng.uniform(-3, 2.5, 5000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(si.fp8_e4m3_round_bits(x), ref)


def test_encoder_saturates():
    assert list(si.fp8_e4m3_round_bits(np.array([460.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0xFE]


def test_quantize_maps_amax_to_max_code():
    rng = np.random.default_rng(3)
    codes, descale = si.quantize_fp8(rng, (4, 64))
    vals = fa_oracle.fp8_e4m3_value(codes) * descale
    assert np.abs(codes & 0x7F).max() == 0x7E
    rng = np.random.default_rng(3)
    x = rng.standard_normal(size=(4, 64), dtype=np.float32).astype(np.float64)
    # every value within half a code step (relative 2^-4, or 2^-10 descale near zero)
    tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * descale)
    assert (np.abs(vals - x) <= tol * (1 + 1e-12)).all()


def _fp8_case(rng, B, Hq, Hkv, N, d):
    q, qs = si.quantize_fp8(rng, (B, Hq, N, d))
    k, ks = si.quantize_fp8(rng, (B, Hkv, N, d))
    v, vs = si.quantize_fp8(rng, (B, Hkv, N, d))
    return q, k, v, qs, ks, vs


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ref_matches_torch_sdpa(causal):
    rng = np.random.default_rng(21)
    q, k, v, qs, ks, vs = _fp8_case(rng, 1, 2, 1, 37, 16)
    scale = 0.3
    o, lse = fa_oracle.attention_fp8_ref(q, k, v, qs, ks, vs, causal, scale)
    tq = torch.from_numpy(_torch_decode(q) * qs)
    tk = torch.from_numpy(_torch_decode(k) * ks).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(_torch_decode(v) * vs).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale).numpy()
    assert np.abs(o - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    s = scale * torch.einsum("bhid,bhjd->bhij", tq, tk)
    if causal:
        s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


def test_fp8_ref_closed_forms():
    rng = np.random.default_rng(5)
    q, k, v, qs, ks, vs = _fp8_case(rng, 1, 1, 1, 1, 8)
    o, lse = fa_oracle.attention_fp8_ref(q, k, v, qs, ks, vs, False, 0.5)
    qv = fa_oracle.fp8_e4m3_value(q[0, 0, 0]) * qs
    kv = fa_oracle.fp8_e4m3_value(k[0, 0, 0]) * ks
    assert np.allclose(o[0, 0, 0], fa_oracle.fp8_e4m3_value(v[0, 0, 0]) * vs, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.5 * float(qv @ kv)) <= 1e-13
    # equal keys: O is the mean of V, lse = s + ln N
    N = 50
    q, k, v, qs, ks, vs = _fp8_case(rng, 1, 1, 1, N, 8)
    k[:] = k[:, :, :1]
    o, lse = fa_oracle.attention_fp8_ref(q, k, v, qs, ks, vs, False, 0.25)
    vv = fa_oracle.fp8_e4m3_value(v[0, 0]) * vs
    assert np.abs(o[0, 0] - vv.mean(axis=0)).max() <= 1e-13
    s = 0.25 * (fa_oracle.fp8_e4m3_value(q[0, 0]) * qs) @ (fa_oracle.fp8_e4m3_value(k[0, 0, 0]) * ks)
    assert np.abs(lse[0, 0] - (s + math.log(N))).max() <= 1e-12


def test_fp8_ref_scale_factors():
    """Only the products scale * q_scale * k_scale and v_scale * V matter."""
    rng = np.random.default_rng(6)
    q, k, v, qs, ks, vs = _fp8_case(rng, 1, 2, 2, 40, 16)
    o1, l1 = fa_oracle.attention_fp8_ref(q, k, v, qs, ks, vs, True, 0.2)
    o2, l2 = fa_oracle.attention_fp8_ref(q, k, v, qs * 4, ks / 2, vs * 2, True, 0.1)
    assert np.abs(o2 - 2 * o1).max() <= 1e-14 * np.abs(o1).max() * 4
    assert np.abs(l2 - l1).max() <= 1e-13


def test_decode_pins_catch_planted_mistakes():
    def bias8(c):
        return fa_oracle.fp8_e4m3_value(c) / 2            # exponent bias 8 instead of 7

    def sub10(c):
        v = fa_oracle.fp8_e4m3_value(c)
        e = (np.asarray(c, dtype=np.int64) >> 3) & 15
        return np.where(e == 0, v / 2, v)                  # subnormal step 2^-10

    def nan_at_inf(c):
        v = fa_oracle.fp8_e4m3_value(c)
        e = (np.asarray(c, dtype=np.int64) >> 3) & 15
        return np.where(e == 15, np.nan, v)                # E4M3 with IEEE-style specials

    def no_sign(c):
        return np.abs(fa_oracle.fp8_e4m3_value(c))

    for bad in (bias8, sub10, nan_at_inf, no_sign):
        assert not _decode_pins_hold(bad), bad.__name__
