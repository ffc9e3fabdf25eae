"""The pages' tiled online-softmax algorithm and the split-KV merge, in fp64.

Test infrastructure only (same rule as the rest of ``oracle/``).  This module
is a second reference, written from the algorithm rather than the definition,
so that tests can show on tiny inputs that the tiled method reaches the
definition's result (the pages state it is exact, not an approximation), for
every block size, and that splitting the keys of a query into chunks and
merging the chunk summaries by their log-sum-exp gives the same result.

Sources:
 - "Attention variants: GQA/MQA/FlashAttention" (youngju.dev), §3: Q, K and V
   are cut into blocks; the outer loop walks query blocks, the inner loop key
   and value blocks; per query row a running maximum and running sum are kept
   and the accumulator is brought to the new maximum's scale before a block
   is added; the result equals the untiled attention.  The printed sketch
   leaves the running sum un-updated, keeps one scalar maximum and does not
   define its rescale or finalize helpers: this module takes the standard
   reading, with per-row vectors, l <- l*exp(m-m') + sum exp(s-m') and
   acc <- acc*exp(m-m') + exp(S-m') V, then O = acc / l.
 - §5.5 of the same page: causal key blocks wholly in the future are skipped,
   the diagonal block is masked inside, earlier blocks are used in full.
 - The split-KV merge is not on the pages; it is the same rescale rule applied
   to whole-chunk summaries (m_c + ln l_c, O_c).
"""
from __future__ import annotations

import numpy as np


def _visible(n_q: int, n_k: int, causal: bool) -> np.ndarray:
    """Boolean [n_q, n_k]: key j visible to query i (bottom-right causal)."""
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i + (n_k - n_q)


def tiled_head(q, k, v, scale: float, causal: bool, block_q: int, block_k: int):
    """One head: q [N_q,d], k/v [N_k,d] (fp64) -> (o [N_q,d], lse [N_q])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_q, d = q.shape
    n_k = k.shape[0]
    vis = _visible(n_q, n_k, causal)
    o = np.zeros((n_q, d))
    lse = np.full((n_q,), -np.inf)
    for i0 in range(0, n_q, block_q):                       # outer loop: query blocks
        i1 = min(i0 + block_q, n_q)
        qb = q[i0:i1]
        m = np.full((i1 - i0,), -np.inf)                      # running maximum per row
        l = np.zeros((i1 - i0,))                              # running sum per row
        acc = np.zeros((i1 - i0, d))
        for j0 in range(0, n_k, block_k):                   # inner loop: key/value blocks
            j1 = min(j0 + block_k, n_k)
            vb = vis[i0:i1, j0:j1]
            if not vb.any():                                  # block wholly in the future
                continue
            s = scale * (qb @ k[j0:j1].T)
            s = np.where(vb, s, -np.inf)                      # diagonal block: mask inside
            m_new = np.maximum(m, s.max(axis=1))
            base = np.where(np.isneginf(m_new), 0.0, m_new)   # rows still empty keep 0
            alpha = np.exp(m - base)
            p = np.exp(s - base[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j1]
            m = m_new
        nz = l > 0
        o[i0:i1][nz] = acc[nz] / l[nz, None]
        lse[i0:i1][nz] = m[nz] + np.log(l[nz])
    return o, lse


def split_partials(q, k, v, scale: float, num_splits: int):
    """One query row against n keys, cut into num_splits chunks of ceil(n/S).

    Returns per-chunk (o_c [S,d], lse_c [S]); an empty chunk has lse_c = -inf
    and o_c = 0.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = k.shape
    chunk = -(-n // num_splits)
    o_c = np.zeros((num_splits, d))
    lse_c = np.full((num_splits,), -np.inf)
    for c in range(num_splits):
        j0, j1 = c * chunk, min((c + 1) * chunk, n)
        if j0 >= j1:
            continue
        s = scale * (k[j0:j1] @ q)
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        o_c[c] = (p @ v[j0:j1]) / l
        lse_c[c] = m + np.log(l)
    return o_c, lse_c


def merge_partials(o_c, lse_c):
    """LSE merge of chunk summaries: M = max lse_c, lse = M + ln sum exp(lse_c - M),
    o = sum exp(lse_c - lse) o_c."""
    o_c = np.asarray(o_c, np.float64)
    lse_c = np.asarray(lse_c, np.float64)
    mx = lse_c.max()
    if np.isneginf(mx):
        return np.zeros(o_c.shape[1]), -np.inf
    w = np.exp(lse_c - mx)
    lse = mx + np.log(w.sum())
    o = (np.exp(lse_c - lse)[:, None] * o_c).sum(axis=0)
    return o, lse
