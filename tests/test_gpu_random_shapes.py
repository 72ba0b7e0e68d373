"""Seeded random shapes through every entry point, against the FP64 oracle.

The other parity tests choose their shapes by hand (the workloads, the edges,
each planner path). This module draws further shapes from a fixed seed: batch,
query and KV head counts (any group size that divides), sequence length,
head dimension, mask and scale (1/sqrt(d) times 1/2, 1 or 2). Every draw is
deterministic, and all are small enough for the oracle to check every row. The
forward, FP8 forward, backward and decode (uniform and variable length) each
take their own draws and run through the same checks and gates as their
dedicated tests.
"""
import math

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import have_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _draw(seed: int, count: int, n_max: int):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4]))
        while hkv * g > 8:
            g //= 2
        d = int(rng.choice([64, 128]))
        out.append(dict(B=int(rng.integers(1, 3)), Hq=hkv * g, Hkv=hkv, N=int(rng.integers(1, n_max + 1)), d=d,
                        causal=bool(rng.integers(2)), scale=float(rng.choice([0.5, 1.0, 2.0])) / math.sqrt(d),
                        seed=int(rng.integers(1 << 30))))
    return out


def _id(s):
    return f"B{s['B']}_H{s['Hq']}-{s['Hkv']}_N{s['N']}_d{s['d']}_{'c' if s['causal'] else 'n'}_s{s['scale'] * math.sqrt(s['d']):g}"


FWD = _draw(8101, 12, 1500)
FP8 = _draw(8102, 8, 1500)
BWD = _draw(8103, 8, 700)
DEC = _draw(8104, 8, 3000)


@pytest.mark.parametrize("s", FWD, ids=_id)
def test_fwd_random(s):
    from test_gpu_fwd import _run_case
    case = si.FwdCase("random " + _id(s), s["B"], s["Hq"], s["Hkv"], s["N"], s["d"], s["causal"], s["seed"])
    _run_case(case, scale=s["scale"])


@pytest.mark.parametrize("s", FP8, ids=_id)
def test_fwd_fp8_random(s):
    from test_gpu_fwd_fp8 import _run
    _run("random fp8 " + _id(s), s["B"], s["Hq"], s["Hkv"], s["N"], s["causal"], s["seed"], scale=s["scale"],
         d=s["d"])


@pytest.mark.parametrize("s", BWD, ids=_id)
def test_bwd_random(s):
    from test_gpu_bwd import _run_small
    _run_small(s["B"], s["Hq"], s["Hkv"], s["N"], s["causal"], s["seed"], scale=s["scale"], d=s["d"])


@pytest.mark.parametrize("s", DEC, ids=_id)
def test_decode_random(s):
    """Decode with the draw's N as the cache length and a split count drawn in 1..min(32, L); the odd
    draws also give each sequence a length in 0..L (the variable-length entry point)."""
    from test_gpu_decode import _run, _run_varlen
    rng = np.random.default_rng(s["seed"])
    L = s["N"]
    splits = int(rng.integers(1, min(32, L) + 1))
    if s["causal"]:  # the draw's mask bit picks the variable-length form
        lens = [int(x) for x in rng.integers(0, L + 1, size=s["B"])]
        _run_varlen("random varlen " + _id(s), s["B"], s["Hq"], s["Hkv"], L, s["d"], splits, lens, s["seed"])
    else:
        _run(si.DecodeCase("random " + _id(s), s["B"], s["Hq"], s["Hkv"], L, s["d"], splits, seed=s["seed"]),
             scale=s["scale"])
