"""Analytic byte, FLOP and footprint models printed on the pages: TEST INFRASTRUCTURE ONLY.

Each function restates, in plain arithmetic, a count the pages derive; the
CPU tests check every printed number against these functions to the printed
rounding. MiB/GiB are binary (2^20, 2^30 bytes), MB and TB/s decimal, as the
"FlashAttention HBM bytes, one head, 8K" page insists ("Common mistakes").
"""
from __future__ import annotations

MiB = 1 << 20
GiB = 1 << 30


# ------------------- "FlashAttention HBM bytes, one head, 8K" (A strong answer)

def tensor_bytes(N: int, d: int, elem: int = 2) -> int:
    """One N x d tensor (BF16 by default)."""
    return N * d * elem


def compulsory_bytes(N: int, d: int, elem: int = 2) -> int:
    """Read Q, K, V and write O once each: the floor for any kernel."""
    return 4 * tensor_bytes(N, d, elem)


def naive_bytes(N: int, d: int, score_elem: int = 2, elem: int = 2) -> int:
    """Unfused attention: write S, read S, write P, read P, plus the compulsory tensors."""
    return 4 * N * N * score_elem + compulsory_bytes(N, d, elem)


def paper_model_bytes(N: int, d: int, block_rows: int, elem: int = 2) -> int:
    """FA2 loop order with every K/V tile load counted as an HBM access.

    N / B_r query blocks each stream all of K and V; Q is read and O written once.
    """
    t_r = N // block_rows
    return t_r * 2 * tensor_bytes(N, d, elem) + 2 * tensor_bytes(N, d, elem)


def fwd_flops(N: int, d: int, causal: bool = False) -> float:
    """4 N^2 d for QK^T and PV; causal skips the masked tiles and halves it."""
    f = 4.0 * N * N * d
    return f / 2 if causal else f


def decode_kv_bytes(L: int, d: int, elem: int = 2) -> int:
    """Decode reads K and V once per KV head."""
    return 2 * L * d * elem


def decode_flops(L: int, d: int) -> float:
    """One query against L keys: 4 L d FLOPs per query head."""
    return 4.0 * L * d


def decode_intensity(L: int, d: int, group: int) -> float:
    """FLOP per byte of K/V for a GQA group sharing one KV head."""
    return group * decode_flops(L, d) / decode_kv_bytes(L, d)


# ------------- "Flash Attention Mechanics: How Tiled Attention Fits in SRAM"

def standard_footprint_gib(N: int, heads: int, d: int, elem: int = 2) -> dict:
    """Standard attention's resident memory: the score matrix plus Q, K, V and O."""
    scores = heads * N * N * elem / GiB
    qkv = 3 * heads * N * d * elem / GiB
    out = heads * N * d * elem / GiB
    return {"scores": scores, "qkv": qkv, "out": out, "total": scores + qkv + out}


def flash_footprint_gib(N: int, heads: int, d: int, elem: int = 2) -> dict:
    """FlashAttention's resident memory: Q, K, V, O plus two statistics per row.

    The page's footprint function sizes the statistics with the same 2-byte
    element as the tensors.
    """
    qkvo = 4 * heads * N * d * elem / GiB
    stats = heads * N * 2 * elem / GiB
    return {"qkvo": qkvo, "stats": stats, "total": qkvo + stats}


def hbm_traffic_gib(N: int, heads: int, d: int, elem: int = 2) -> dict:
    """Forward HBM traffic: standard = four passes over S plus Q, K, V, O; flash = Q, K, V, O."""
    score_pass = heads * N * N * elem
    qkvo = 4 * heads * N * d * elem
    std = (4 * score_pass + qkvo) / GiB
    fl = qkvo / GiB
    return {"standard": std, "flash": fl, "reduction": std / fl}


def sram_usage_kib(block: int, d: int, elem: int = 2) -> dict:
    """On-chip bytes for square blocks: Q, K, V, O tiles plus FP32 m and l per row."""
    q = block * d * elem / 1024
    kv = 2 * block * d * elem / 1024
    o = block * d * elem / 1024
    stats = block * 2 * 4 / 1024
    return {"q": q, "kv": kv, "out": o, "stats": stats, "total": q + kv + o + stats}


def tile_intensity(block: int, d: int, elem: int = 2) -> float:
    """FLOPs of one tile step (QK^T and PV) per byte of K and V tile loaded."""
    return (4.0 * block * block * d) / (2 * block * d * elem)


def best_block(sram_kib: float, d: int, candidates=(16, 32, 64, 128, 256, 512)) -> int:
    """Largest candidate block whose tiles and statistics fit the on-chip budget."""
    fits = [b for b in candidates if sram_usage_kib(b, d)["total"] <= sram_kib]
    return max(fits) if fits else 0


# ------ "Why is standard attention memory-bound, and how does FlashAttention fix it?"

def machine_balance(flops_per_s: float, bytes_per_s: float) -> float:
    """Peak FLOP/s over memory bytes/s."""
    return flops_per_s / bytes_per_s


def standard_traffic_bytes(N: int, d: int, elem: int = 2) -> int:
    """Four passes over the N x N matrix plus Q, K, V and O, one head."""
    return 4 * N * N * elem + 4 * N * d * elem


def tiled_kv_block(sram_numbers: int, d: int) -> int:
    """Column block from an on-chip budget counted in numbers: M / (4 d)."""
    return sram_numbers // (4 * d)


def tiled_traffic_bytes(N: int, d: int, block_cols: int, elem: int = 2) -> int:
    """Tiled traffic with K/V blocks in the outer loop, one head.

    Reading: each of the N / B_c outer passes reads Q and the partial O and
    writes O back (3 N d elements); K and V are read once overall (2 N d).
    This reproduces the page's 26.2 MB and 102.8 MB figures.
    """
    passes = N // block_cols
    return passes * 3 * N * d * elem + 2 * N * d * elem
