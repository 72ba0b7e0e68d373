"""FP64 CPU oracle for exact attention: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the bench's CPU-baseline leg use this module;
the HIP library shares no code with it. Everything here is the plain
definition, computed in float64 on BF16-valued inputs (widened exactly), with
the N x N score matrix S and the weight matrix P materialised, exactly as the
unfused "standard attention" the pages describe:

  * "Flash Attention Mechanics: How Tiled Attention Fits in SRAM", section
    "Why Standard Attention Is Memory-Bound": O = softmax(Q K^T / sqrt(d)) V,
    with the full score matrix materialised ("standard attention" listing in
    "The Tiling Algorithm").
  * "Why is standard attention memory-bound, and how does FlashAttention fix
    it?", "Step 1": three passes -- S = Q K^T, P = softmax(S), O = P V.
  * "FlashAttention HBM bytes, one head, 8K", "A strong answer" (Naive): the
    same three unfused passes.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * scale is a caller argument; the workloads pass 1/sqrt(d).
  * lse is the natural log of sum_j exp(scale * q.k_j) (it includes the scale).
  * causal means key j is visible to query i iff j <= i (square, N_q = N_k).
  * a row with no visible key has O = 0 and lse = -inf (unreachable through
    the library's argument checks, defined here for completeness).
  * GQA: query head h reads KV head h // (Hq // Hkv).

The FP8 variant (attention_fp8_ref) is the same definition applied to the
values of OCP FP8 E4M3 codes times per-tensor factors (fp8_e4m3_value decodes
the codes from the format's bit layout).

Parity: every function here is pinned by the CPU test-suite (the printed toy
run of the online softmax, closed forms, invariants, brute force on tiny
inputs and torch's FP64 CPU scaled_dot_product_attention).
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 256  # rows per materialised S block (bounds memory to 256 x N x 8 B)


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _standard_attention_rows(qr: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                             row_ids: np.ndarray | None, causal: bool):
    """Three unfused passes for a block of query rows of one head.

    qr: [R, d] query rows; k, v: [N, d]; row_ids: the global index of each row
    (needed for the causal mask). Returns (O [R, d], lse [R], P [R, N]).
    """
    # Pass 1: scores S = scale * Q K^T, materialised.
    s = scale * (qr @ k.T)
    if causal:
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols <= row_ids[:, None], s, -np.inf)
    # Pass 2: P = softmax(S) row by row (max-subtracted for range, then normalised).
    m = s.max(axis=1)
    dead = ~np.isfinite(m)  # rows with no visible key
    m_safe = np.where(dead, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    l_safe = np.where(dead, 1.0, l)
    p = p / l_safe[:, None]
    # Pass 3: O = P V.
    o = p @ v
    lse = np.where(dead, -np.inf, m_safe + np.log(l_safe))
    o[dead] = 0.0
    return o, lse, p


def _rows_for_head(rows, h: int, N: int) -> np.ndarray:
    if rows is None:
        return np.arange(N, dtype=np.int64)
    r = np.asarray(rows, dtype=np.int64)
    if r.ndim == 1:
        return r
    return r[h]


def attention_ref(q, k, v, causal: bool, scale: float, rows=None, return_p: bool = False):
    """Exact attention O = softmax(scale Q K^T) V and its per-row logsumexp.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype; computed in FP64).
    rows: None for every row, a 1-D array of row indices used for every head,
    or a 2-D array [Hq, R] of per-head rows.
    Returns O [B, Hq, R, d] and lse [B, Hq, R] (float64; natural log), plus
    P [B, Hq, R, N] when ``return_p`` (small inputs only).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    R = len(_rows_for_head(rows, 0, N))
    dv = v.shape[-1]  # V may be wider or narrower than Q/K (used by one-hot probes)
    o_out = np.zeros((B, Hq, R, dv))
    lse_out = np.zeros((B, Hq, R))
    p_out = np.zeros((B, Hq, R, k.shape[2])) if return_p else None
    for b in range(B):
        for h in range(Hq):
            kh = _as_f64(k[b, h // group])
            vh = _as_f64(v[b, h // group])
            rid = _rows_for_head(rows, h, N)
            for c0 in range(0, R, ROW_CHUNK):
                ids = rid[c0:c0 + ROW_CHUNK]
                qr = _as_f64(q[b, h, ids])
                o, lse, p = _standard_attention_rows(qr, kh, vh, scale, ids, causal)
                o_out[b, h, c0:c0 + len(ids)] = o
                lse_out[b, h, c0:c0 + len(ids)] = lse
                if return_p:
                    p_out[b, h, c0:c0 + len(ids)] = p
    if return_p:
        return o_out, lse_out, p_out
    return o_out, lse_out


def attention_bwd_ref(q, k, v, do, causal: bool, scale: float, rows=None, key_rows=None):
    """Gradients of the exact attention of attention_ref, contracted with dO.

    "Why is standard attention memory-bound, and how does FlashAttention fix
    it?" ("Step 4: The result is exact, and the backward pass recomputes"; FAQ
    "Why does the backward pass recompute the scores?"): the backward pass
    needs the scores, which FlashAttention recomputes tile by tile from Q, K and
    the saved per-row statistics. The pages state no formulas; this is the
    plain chain rule through O = P V, P = softmax(S), S = scale Q K^T, with S,
    P, dP and dS materialised (row chunks of all query rows):

        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.

    GQA: the gradients of a KV head sum over the query heads that read it.
    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d]. rows / key_rows select the
    query rows of dQ and the key rows of dK, dV (None: all; 1-D: the same for
    every head; 2-D: per query head / per KV head). Returns dQ [B, Hq, R, d],
    dK [B, Hkv, Rk, d], dV [B, Hkv, Rk, dv] in float64.
    """
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    R = len(_rows_for_head(rows, 0, N))
    Rk = len(_rows_for_head(key_rows, 0, N))
    dvw = v.shape[-1]
    dq_out = np.zeros((B, Hq, R, d))
    dk_out = np.zeros((B, Hkv, Rk, d))
    dv_out = np.zeros((B, Hkv, Rk, dvw))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            kh, vh = _as_f64(k[b, g]), _as_f64(v[b, g])
            rid = _rows_for_head(rows, h, N)
            kid = _rows_for_head(key_rows, g, N)
            where = {int(r): n for n, r in enumerate(rid)}
            for c0 in range(0, N, ROW_CHUNK):
                ids = np.arange(c0, min(N, c0 + ROW_CHUNK))
                qr, dor = _as_f64(q[b, h, ids]), _as_f64(do[b, h, ids])
                _, _, p = _standard_attention_rows(qr, kh, vh, scale, ids, causal)
                dp = dor @ vh.T
                dsum = (p * dp).sum(axis=1)
                ds = p * (dp - dsum[:, None])
                dv_out[b, g] += p[:, kid].T @ dor
                dk_out[b, g] += scale * (ds[:, kid].T @ qr)
                for n_local, r in enumerate(ids):
                    if int(r) in where:
                        dq_out[b, h, where[int(r)]] = scale * (ds[n_local] @ kh)
    return dq_out, dk_out, dv_out


def decode_ref(q, k, v, scale: float):
    """One query token per (sequence, query head) against the whole KV cache.

    The decode follow-up of "FlashAttention HBM bytes, one head, 8K" ("What
    interviewers probe next") and "Does FlashAttention help when generating one
    token at a time?" on the memory-bound page: same definition, one row, no
    mask. q: [B, Hq, d] or [B, Hq, 1, d]; k, v: [B, Hkv, L, d].
    Returns O [B, Hq, d] and lse [B, Hq].
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    o_out = np.zeros((B, Hq, np.asarray(v).shape[-1]))
    lse_out = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            o, lse, _ = _standard_attention_rows(_as_f64(q[b, h])[None, :], _as_f64(k[b, h // group]),
                                                 _as_f64(v[b, h // group]), scale, None, False)
            o_out[b, h] = o[0]
            lse_out[b, h] = lse[0]
    return o_out, lse_out


def decode_varlen_ref(q, k, v, lens, scale: float):
    """decode_ref for a batch of KV caches of their own lengths.

    Sequence b attends to keys 0 .. len_b - 1 of its (padded) cache rows, with
    len_b = lens[b] clamped to [0, L]; the padding takes no part. A sequence
    with no key has an empty sum: O = 0 and lse = ln 0 = -inf (the defined
    output for a row with every key masked).
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, _ = q.shape
    L = np.asarray(k).shape[2]
    o_out = np.zeros((B, Hq, np.asarray(v).shape[-1]))
    lse_out = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), L))
        if n == 0:
            continue
        o, lse = decode_ref(q[b:b + 1], np.asarray(k)[b:b + 1, :, :n], np.asarray(v)[b:b + 1, :, :n], scale)
        o_out[b], lse_out[b] = o[0], lse[0]
    return o_out, lse_out


def split_chunks(L: int, num_splits: int):
    """Key ranges of a split-KV decode: chunk = ceil(L / num_splits) keys each."""
    chunk = -(-L // num_splits)
    return [(c * chunk, min(L, (c + 1) * chunk)) for c in range(num_splits)]


def split_decode_partials_ref(q, k, v, scale: float, num_splits: int):
    """Per-chunk partial results of split-KV decode, each by the plain definition.

    For chunk c with keys [a, b): O_c = softmax over those keys only, applied
    to their V rows; lse_c = log sum over those keys of exp(scale q.k). An
    empty chunk has O_c = 0 and lse_c = -inf.
    Returns O_parts [B, Hq, S, d] and lse_parts [B, Hq, S].
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, d = q.shape
    L = k.shape[2]
    chunks = split_chunks(L, num_splits)
    o_parts = np.zeros((B, Hq, num_splits, np.asarray(v).shape[-1]))
    lse_parts = np.full((B, Hq, num_splits), -np.inf)
    for c, (a, e) in enumerate(chunks):
        if e <= a:
            continue
        o, lse = decode_ref(q, np.asarray(k)[:, :, a:e], np.asarray(v)[:, :, a:e], scale)
        o_parts[:, :, c] = o
        lse_parts[:, :, c] = lse
    return o_parts, lse_parts


def combine_ref(o_parts, lse_parts):
    """Log-sum-exp merge of normalised partial results over disjoint key sets.

    This is the merge step of the online softmax ("The Tiling Algorithm" on the
    Flash Attention Mechanics page; "Step 3" on the memory-bound page) applied
    to whole chunks: with M = max_c lse_c and w_c = exp(lse_c - M),
    O = sum_c w_c O_c / sum_c w_c and lse = M + log sum_c w_c.
    o_parts: [..., S, d]; lse_parts: [..., S]. Chunks with lse = -inf carry no
    weight; if every chunk is empty, O = 0 and lse = -inf.
    """
    o_parts = _as_f64(o_parts)
    lse_parts = _as_f64(lse_parts)
    m = lse_parts.max(axis=-1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    w = np.exp(lse_parts - m_safe[..., None])
    wsum = w.sum(axis=-1)
    wsum_safe = np.where(dead, 1.0, wsum)
    o = (w[..., None] * o_parts).sum(axis=-2) / wsum_safe[..., None]
    o[dead] = 0.0
    lse = np.where(dead, -np.inf, m_safe + np.log(wsum_safe))
    return o, lse


def fp8_e4m3_value(codes) -> np.ndarray:
    """The value of each OCP FP8 E4M3 code (uint8), in float64.

    Bit layout S.EEEE.MMM with exponent bias 7: E = 0 holds the subnormals
    M 2^-9 (and signed zeros), E = 1..15 holds (1 + M/8) 2^(E-7), and
    S.1111.111 is NaN (the format has no infinity, so E = 15 with M < 7 is
    still finite: up to 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def attention_fp8_ref(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, causal: bool,
                      scale: float, rows=None, return_p: bool = False):
    """Exact attention of FP8-coded inputs with per-tensor dequantisation factors.

    The 8-bit variant named in "Why is standard attention memory-bound, and how
    does FlashAttention fix it?" ("What does FlashAttention-2 change?": the third
    version adds FP8 low precision) changes the input format, not the result
    being approximated: the inputs are the values q_scale * Q, k_scale * K and
    v_scale * V of the E4M3 codes, and O and lse are the exact attention of
    those values (attention_ref, in FP64).
    """
    q = fp8_e4m3_value(q8) * float(q_scale)
    k = fp8_e4m3_value(k8) * float(k_scale)
    v = fp8_e4m3_value(v8) * float(v_scale)
    return attention_ref(q, k, v, causal, scale, rows=rows, return_p=return_p)
