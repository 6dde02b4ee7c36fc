"""Softmax attention restricted to kept N x N blocks, fp64 (test infrastructure only).

Source: the FlashAttention abstract (Daily Papers listing) extends exact tiled
attention to block-sparse attention that computes only the listed blocks; the
related-paper listing states that online softmax is exact. The result is therefore
the plain definition: for query token p, key token q is allowed iff the block pair
(p // N, q // N) is kept and q < S_valid; O_p = sum_q softmax_q(scale * <Q_p, K_q>) V_q
over allowed q. Conventions (design notes): a query with no allowed key, and every
padded query row p >= S_valid, gets O_p = 0 and lse = -inf.
"""
import numpy as np


def block_sparse_attention(q, k, v, block_mask, n: int, s_valid: int, scale=None,
                           q_blocks=None):
    """One head. q, k, v [S, D]; block_mask bool [S/n, S/n].

    Returns (O [S, D] float64, lse [S] float64, natural log). Rows of query blocks
    not listed in `q_blocks` (default: all) are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb = S // n
    O = np.full((S, D), np.nan)
    lse = np.full(S, np.nan)
    blocks = range(nb) if q_blocks is None else q_blocks
    for i in blocks:
        rows = np.arange(i * n, (i + 1) * n)
        O[rows] = 0.0
        lse[rows] = -np.inf
        rows = rows[rows < s_valid]
        kept = np.nonzero(block_mask[i])[0]
        cols = np.concatenate([np.arange(j * n, (j + 1) * n) for j in kept]) if len(kept) \
            else np.zeros(0, dtype=np.int64)
        cols = cols[cols < s_valid]
        if len(rows) == 0 or len(cols) == 0:
            continue
        s = scale * (q[rows] @ k[cols].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[rows] = (e @ v[cols]) / l
        lse[rows] = (m + np.log(l))[:, 0]
    return O, lse
