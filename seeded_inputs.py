"""Seeded synthetic inputs for exact tiled attention.

This module is the only code shared by the HIP path's callers (tests, bench,
smoke) and the CPU oracle. It draws random numbers and rounds them to BF16; it
holds none of the attention arithmetic.

Workloads follow the shapes the three source pages use:
  * "FlashAttention HBM bytes, one head, 8K" (one head, N=8192, d=128, BF16,
    with causal and GQA-decode follow-ups),
  * "Flash Attention Mechanics" (32 heads, d=128; a seq-1024, d-64 harness),
  * "Why is standard attention memory-bound" (one head, N=4096/8192).
Values are i.i.d. N(0,1) drawn in float32 with numpy's PCG64 generator
(``np.random.default_rng(seed)``), in the order Q, K, V, then rounded to the
nearest BF16 (ties to even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# ---------------------------------------------------------------- BF16 bits

def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); return uint16 bits.

    NaN stays a quiet NaN; infinities and overflow to infinity follow IEEE RNE.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bits to float32 exactly (the BF16 value is a float32 prefix)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """One N(0,1) float32 draw of ``shape`` rounded to BF16 bits."""
    return bf16_round_bits(rng.standard_normal(size=shape, dtype=np.float32))


# ---------------------------------------------------------------- FP8 E4M3 bits

FP8_E4M3_MAX = 448.0  # largest finite OCP E4M3 value (1.75 x 2^8)


def fp8_e4m3_round_bits(x: np.ndarray) -> np.ndarray:
    """Round values to OCP FP8 E4M3 ("E4M3FN": 4 exponent bits, bias 7, 3
    mantissa bits, subnormals, no infinity, NaN = S.1111.111); nearest, ties
    to even; magnitudes above 448 saturate to 448. Returns uint8 codes.

    Normal codes hold (1 + m/8) 2^(e-7) for e = 1..15; subnormal codes hold
    m 2^-9 for e = 0, so the subnormal step 2^-9 continues into the first
    normal binade and one rounding rule covers both.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    sign = np.signbit(x).astype(np.uint8) << 7
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))           # binade (>= -6: subnormals share it)
    step = 2.0 ** (e - 3)                                      # spacing of codes in that binade
    k = np.rint(a / step)                                      # ties to even
    e = np.where(k >= 16, e + 1, e)                            # rounded up into the next binade
    k = np.where(k >= 16, k / 2, k)
    normal = k >= 8
    code = np.where(normal, ((e + 7).astype(np.int64) << 3) | (k.astype(np.int64) - 8),
                    k.astype(np.int64))
    code = np.where(np.isnan(x), 0x7F, code)
    return (code.astype(np.uint8) | np.where(np.isnan(x), 0, sign)).astype(np.uint8)


def quantize_fp8(rng: np.random.Generator, shape):
    """One N(0,1) float32 draw quantised per tensor: (codes, descale) with the
    values codes * descale and descale = max|x| / 448 (so max|x| maps to 448)."""
    x = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    amax = float(np.abs(x).max()) if x.size else 1.0
    descale = np.float32(amax / FP8_E4M3_MAX if amax > 0 else 1.0)
    return fp8_e4m3_round_bits(x / float(descale)), float(descale)


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class FwdCase:
    """A forward workload: Q,O [B,Hq,N,d]; K,V [B,Hkv,N,d]; all BF16."""
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    sampled_rows: int | None = None  # rows per head the oracle checks (None = all)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    """A decode workload: Q,O [B,Hq,1,d]; K,V [B,Hkv,L,d]; split-KV."""
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    num_splits: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads. Seeds 1..5 in order.
TINY = FwdCase("1x1x128 d64", 1, 1, 1, 128, 64, False, seed=1)
ONE_HEAD_8K = FwdCase("1x1x8192 d128", 1, 1, 1, 8192, 128, False, seed=2)
ONE_HEAD_8K_CAUSAL = dataclasses.replace(ONE_HEAD_8K, name="1x1x8192 d128 causal", causal=True)
HEADS32_4K = FwdCase("1x32x4096 d128", 1, 32, 32, 4096, 128, False, seed=3, sampled_rows=1024)
HEADS32_4K_CAUSAL = dataclasses.replace(HEADS32_4K, name="1x32x4096 d128 causal", causal=True)
LONG_128K = FwdCase("1x8x131072 d128 causal", 1, 8, 8, 131072, 128, True, seed=4, sampled_rows=1024)
DECODE_GQA = DecodeCase("decode B16 Hq32 Hkv8 L8192 d128 s16", 16, 32, 8, 8192, 128, 16, seed=5)


def fwd_inputs(case: FwdCase):
    """(q, k, v) BF16 bit arrays for a forward workload, drawn Q, K, V in order."""
    rng = np.random.default_rng(case.seed)
    q = normal_bf16(rng, (case.B, case.Hq, case.N, case.d))
    k = normal_bf16(rng, (case.B, case.Hkv, case.N, case.d))
    v = normal_bf16(rng, (case.B, case.Hkv, case.N, case.d))
    return q, k, v


def fwd_fp8_inputs(case: FwdCase):
    """(q, k, v, q_scale, k_scale, v_scale): FP8 E4M3 code arrays of a forward
    workload's shapes and their per-tensor dequantisation factors, drawn Q, K,
    V in order (N(0,1) float32, each scaled so its largest magnitude is 448)."""
    rng = np.random.default_rng(case.seed)
    q, qs = quantize_fp8(rng, (case.B, case.Hq, case.N, case.d))
    k, ks = quantize_fp8(rng, (case.B, case.Hkv, case.N, case.d))
    v, vs = quantize_fp8(rng, (case.B, case.Hkv, case.N, case.d))
    return q, k, v, qs, ks, vs


def decode_inputs(case: DecodeCase):
    """(q, k, v) BF16 bit arrays for a decode workload: q [B,Hq,1,d]."""
    rng = np.random.default_rng(case.seed)
    q = normal_bf16(rng, (case.B, case.Hq, 1, case.d))
    k = normal_bf16(rng, (case.B, case.Hkv, case.L, case.d))
    v = normal_bf16(rng, (case.B, case.Hkv, case.L, case.d))
    return q, k, v


def sample_rows(seed: int, head: int, N: int, count: int, boundary: int = 64) -> np.ndarray:
    """Sorted seeded sample of ``count`` query rows for one head.

    Rows 0 and N-1 and the rows on each side of a few ``boundary``-multiples
    are always included; the rest are drawn without replacement from
    ``default_rng(seed*1000 + head)``.
    """
    if count >= N:
        return np.arange(N, dtype=np.int64)
    forced = {0, N - 1}
    for t in (1, 2, N // (2 * boundary), N // boundary - 1):
        c = t * boundary
        if 0 < c < N:
            forced.update((c - 1, c))
    forced = sorted(r for r in forced if 0 <= r < N)[:count]
    rng = np.random.default_rng(seed * 1000 + head)
    pool = np.setdiff1d(np.arange(N, dtype=np.int64), np.array(forced, dtype=np.int64))
    extra = rng.choice(pool, size=count - len(forced), replace=False)
    return np.sort(np.concatenate([np.array(forced, dtype=np.int64), extra]))


def growing_score_inputs(N: int, d: int, H: int = 2, seed: int = 1500):
    """Q with first component 4 and K with first component 0.4 j sqrt(d/128)
    (N(0,1) elsewhere), float32: at scale 1/sqrt(d) the scores of a row grow
    by about 10 in base 2 per 64 keys, so a running maximum taken 64 keys at
    a time rises on every step."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, N, d), dtype=np.float32)
    k = rng.standard_normal((1, H, N, d), dtype=np.float32)
    v = rng.standard_normal((1, H, N, d), dtype=np.float32)
    q[..., 0] = 4.0
    k[..., 0] = 0.4 * np.arange(N, dtype=np.float32)[None, None, :] * math.sqrt(d / 128.0)
    return q, k, v
