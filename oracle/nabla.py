"""NABLA adaptive block mask in fp64 (test infrastructure only).

Source: the Pith review of "NABLA: Neighborhood Adaptive Block-Level Attention"
(arXiv 2507.13546), sections "What carries the argument" and "Core claim", and the
referee report's minor comment 2 on Algorithm 1. Per head:
  1. cut Q and K into N-token blocks and average each block to one vector;
  2. reduced map L = scale * Qbar Kbar^T, an (S/N) x (S/N) matrix;
  3. softmax each row of L;
  4. along the key-block axis, sort each row by descending probability, take the
     cumulative sum, and keep the smallest prefix whose mass reaches 1 - thr;
  5. write the binary result back in the original key-block order.

Readings where the text is silent (each listed in the design notes):
  * "smallest prefix reaching 1 - thr" means: in sorted order, entry r is kept iff
    the mass strictly before it, E_r, is < 1 - thr; the top entry is always kept;
  * ties in probability are broken by ascending key-block index;
  * scale defaults to 1/sqrt(D), the usual attention temperature;
  * zero padding at the end of the sequence is pooled as is (divide by N).
"""
import numpy as np


def block_pool(x: np.ndarray, n: int) -> np.ndarray:
    """Mean of each run of n consecutive rows: [S, D] -> [S/n, D] (step 1)."""
    x = np.asarray(x, dtype=np.float64)
    S, D = x.shape
    if S % n:
        raise ValueError("S must be a multiple of the block size")
    return x.reshape(S // n, n, D).sum(axis=1) / n


def reduced_map(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """L[i, j] = scale * <qbar_i, kbar_j> (step 2)."""
    return scale * (qbar @ kbar.T)


def row_softmax(L: np.ndarray) -> np.ndarray:
    """Softmax along each row, with the row maximum subtracted first (step 3)."""
    e = np.exp(L - L.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def cdf_select(P: np.ndarray, thr: float):
    """Steps 4-5 on a matrix of row distributions P [rows, nb].

    Returns (keep bool [rows, nb], E float64 [rows, nb]) where E[i, j] is the mass
    of the entries that precede j in row i's descending order, i.e. the exclusive
    cumulative sum read back in the original column order.
    """
    rows, nb = P.shape
    col = np.broadcast_to(np.arange(nb), P.shape)
    order = np.lexsort((col, -P), axis=1)          # descending p, then ascending index
    p_sorted = np.take_along_axis(P, order, axis=1)
    incl = np.cumsum(p_sorted, axis=1)              # sequential left-to-right sum
    excl = np.zeros_like(incl)
    excl[:, 1:] = incl[:, :-1]
    keep_sorted = excl < (1.0 - thr)
    keep = np.zeros((rows, nb), dtype=bool)
    E = np.zeros((rows, nb))
    np.put_along_axis(keep, order, keep_sorted, axis=1)
    np.put_along_axis(E, order, excl, axis=1)
    return keep, E


def topk_select(P: np.ndarray, topk: int) -> np.ndarray:
    """The fixed-count alternative the NABLA review compares CDF thresholding with
    (Appendix C, Theorem 1: CDF vs Top-k at equal retained blocks): keep the topk
    entries of each row in the same descending order (ties by ascending index)."""
    rows, nb = P.shape
    col = np.broadcast_to(np.arange(nb), P.shape)
    order = np.lexsort((col, -P), axis=1)
    keep_sorted = np.zeros((rows, nb), dtype=bool)
    keep_sorted[:, :min(int(topk), nb)] = True
    keep = np.zeros((rows, nb), dtype=bool)
    np.put_along_axis(keep, order, keep_sorted, axis=1)
    return keep


def topk_mask(q: np.ndarray, k: np.ndarray, n: int, topk: int, scale=None):
    """One head: the reduced map of `nabla_mask`, rows cut to their topk largest entries."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    P = row_softmax(reduced_map(block_pool(q, n), block_pool(k, n), scale))
    return topk_select(P, topk), P


def nabla_mask(q: np.ndarray, k: np.ndarray, n: int, thr: float, scale=None):
    """One head: q, k [S, D] -> (keep bool [nb, nb], E [nb, nb], P [nb, nb])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    P = row_softmax(reduced_map(block_pool(q, n), block_pool(k, n), scale))
    keep, E = cdf_select(P, thr)
    return keep, E, P


def nabla_masks(q, k, n: int, thr: float, scale=None):
    """All heads: q, k [B, H, S, D] -> (keep [B, H, nb, nb], E [B, H, nb, nb])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, S, _ = q.shape
    nb = S // n
    keep = np.zeros((B, H, nb, nb), dtype=bool)
    E = np.zeros((B, H, nb, nb))
    for b in range(B):
        for h in range(H):
            keep[b, h], E[b, h], _ = nabla_mask(q[b, h], k[b, h], n, thr, scale)
    return keep, E
