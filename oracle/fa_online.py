"""FP64 model of the tiled online-softmax algorithm: TEST INFRASTRUCTURE ONLY.

This is the algorithm the pages describe, taken step by step in their order
and notation, so that the CPU tests can show that the tiled algebra (what the
GPU kernels do) and the plain definition in ``fa_oracle`` agree:

  * "Flash Attention Mechanics: How Tiled Attention Fits in SRAM", section
    "The Tiling Algorithm": Q is cut into row blocks, K and V into column
    blocks; for each Q block the running max m = -inf, running sum l = 0 and
    unnormalised output o = 0 are set, every K/V block is swept, and the block's
    statistics are merged; o / l is written at the end.
  * "Why is standard attention memory-bound, and how does FlashAttention fix
    it?", "Step 3" and "What is online softmax?": when a block raises the max
    from m_old to m_new, the running sum and the partial output are multiplied
    by exp(m_old - m_new) before the block's contribution is added.

The causal mask ("What interviewers probe next" on the HBM-bytes page) hides
key j from query i when j > i; a block whose keys are all hidden from a row
contributes nothing to that row.
"""
from __future__ import annotations

import numpy as np


def merge_block(m_old, l_old, o_old, scores_block, v_block):
    """Merge one K/V block into the running (m, l, o) of a block of rows.

    m_old, l_old: [R]; o_old: [R, d]; scores_block: [R, C] (already scaled,
    -inf where masked); v_block: [C, d]. Returns (m_new, l_new, o_new).
    """
    m_blk = scores_block.max(axis=1)
    live = np.isfinite(m_blk)
    m_blk_safe = np.where(live, m_blk, 0.0)
    e = np.exp(scores_block - m_blk_safe[:, None])
    e[~live] = 0.0
    m_new = np.maximum(m_old, np.where(live, m_blk, -np.inf))
    # exp(m_old - m_new) with m_old = m_new = -inf read as 0 (nothing seen yet).
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    a_old = np.where(np.isfinite(m_old), np.exp(m_old - ref), 0.0)
    a_blk = np.where(live, np.exp(m_blk_safe - ref), 0.0)
    l_new = a_old * l_old + a_blk * e.sum(axis=1)
    o_new = a_old[:, None] * o_old + a_blk[:, None] * (e @ v_block)
    return m_new, l_new, o_new


def tiled_attention(q, k, v, scale: float, block_q: int, block_kv: int, causal: bool = False):
    """Tiled exact attention with the online softmax, one head.

    q: [N, d]; k: [N_k, d]; v: [N_k, d_v] (FP64; the causal mask assumes
    N_k = N). Returns O [N, d_v] and lse [N] (natural log).
    Tail blocks are shorter when N is not a multiple of the block size.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[0]
    n_keys = k.shape[0]
    dv = v.shape[1]
    out = np.zeros((N, dv))
    lse = np.zeros(N)
    for q0 in range(0, N, block_q):
        q1 = min(q0 + block_q, N)
        qb = q[q0:q1]
        m = np.full(q1 - q0, -np.inf)
        l = np.zeros(q1 - q0)
        o = np.zeros((q1 - q0, dv))
        for k0 in range(0, n_keys, block_kv):
            k1 = min(k0 + block_kv, n_keys)
            if causal and k0 > q1 - 1:
                break  # every key of this block and beyond is hidden from all rows
            s = scale * (qb @ k[k0:k1].T)
            if causal:
                rows = np.arange(q0, q1)[:, None]
                cols = np.arange(k0, k1)[None, :]
                s = np.where(cols <= rows, s, -np.inf)
            m, l, o = merge_block(m, l, o, s, v[k0:k1])
        out[q0:q1] = o / l[:, None]
        lse[q0:q1] = m + np.log(l)
    return out, lse


def running_stats(scores, blocks):
    """(m, l) of one row after each block of a score sequence.

    ``scores`` is a 1-D list of already-scaled scores and ``blocks`` the list
    of block lengths; l is the running sum of exp(s - m) relative to the
    current running max m. Used to replay the pages' toy run.
    """
    s = np.asarray(scores, dtype=np.float64)
    m = np.array([-np.inf])
    l = np.array([0.0])
    o = np.zeros((1, 1))
    trace = []
    pos = 0
    for n in blocks:
        blk = s[pos:pos + n][None, :]
        m, l, o = merge_block(m, l, o, blk, np.zeros((n, 1)))
        trace.append((float(m[0]), float(l[0])))
        pos += n
    return trace
