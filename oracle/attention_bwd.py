"""Gradients of block-sparse softmax attention, fp64 (test infrastructure only).

Source: the FlashAttention abstract (Daily Papers listing) extends exact tiled
attention, which it uses to train Transformers, to block-sparse attention over the
listed blocks; the NABLA review (Pith review, "Editorial extensions") reports that a
DiT trains with the NABLA block mask, which needs the gradients of attention over
the same mask. No page prints the backward formulas, so this is the plain
derivative of the forward definition in `attention.py`:

    s_pq = scale * <Q_p, K_q> for allowed (p, q), -inf otherwise
    P = row softmax of s,  O = P V,  L = sum_p <dO_p, O_p>
    dV = P^T dO
    dP = dO V^T
    delta_p = sum_q P_pq dP_pq  (= <dO_p, O_p>)
    dS = P * (dP - delta)                     (softmax Jacobian, row by row)
    dQ = scale * dS K,   dK = scale * dS^T Q

with the forward's conventions: key q is allowed for query p iff the block pair
(p // N, q // N) is kept and q < S_valid; padded query rows p >= S_valid and
queries with no allowed key have O_p = 0 independent of every input, so they carry
no gradient (their dQ rows are 0 and they add nothing to dK, dV).
"""
import numpy as np


def block_sparse_attention_bwd(q, k, v, do, block_mask, n: int, s_valid: int, scale=None,
                               q_blocks=None, kv_blocks=None):
    """One head. q, k, v, do [S, D]; block_mask bool [S/n, S/n].

    Returns (dq, dk, dv), each [S, D] float64. dq rows are computed for the query
    blocks in `q_blocks` (default all), dk/dv rows for the key blocks in `kv_blocks`
    (default all); the other rows are NaN. dk/dv of a key block sum over every query
    block that keeps it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    block_mask = np.asarray(block_mask, dtype=bool)
    S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb = S // n
    want_q = set(range(nb)) if q_blocks is None else set(q_blocks)
    want_kv = set(range(nb)) if kv_blocks is None else set(kv_blocks)
    dq = np.full((S, D), np.nan)
    dk = np.full((S, D), np.nan)
    dv = np.full((S, D), np.nan)
    for i in want_q:
        dq[i * n:(i + 1) * n] = 0.0
    for j in want_kv:
        dk[j * n:(j + 1) * n] = 0.0
        dv[j * n:(j + 1) * n] = 0.0
    for i in range(nb):
        kept = np.nonzero(block_mask[i])[0]
        if i not in want_q and not any(j in want_kv for j in kept):
            continue
        rows = np.arange(i * n, (i + 1) * n)
        rows = rows[rows < s_valid]
        cols = np.concatenate([np.arange(j * n, (j + 1) * n) for j in kept]) if len(kept) \
            else np.zeros(0, dtype=np.int64)
        cols = cols[cols < s_valid]
        if len(rows) == 0 or len(cols) == 0:
            continue
        s = scale * (q[rows] @ k[cols].T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        P = e / e.sum(axis=1, keepdims=True)
        O = P @ v[cols]
        dP = do[rows] @ v[cols].T
        delta = np.sum(do[rows] * O, axis=1, keepdims=True)
        dS = P * (dP - delta)
        if i in want_q:
            dq[rows] = scale * (dS @ k[cols])
        sel = np.isin(cols // n, list(want_kv))
        if sel.any():
            # the columns of one row are distinct, so the indexed += adds each once
            dk[cols[sel]] += scale * (dS[:, sel].T @ q[rows])
            dv[cols[sel]] += P[:, sel].T @ do[rows]
    return dq, dk, dv
