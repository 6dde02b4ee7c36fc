"""Shared helpers of the GPU parity tests: oracle reference values and comparisons.

The oracle's functions are called as they are; at the full workload sizes the calls for
different heads or query blocks run on a thread pool (each with single-threaded BLAS),
which changes nothing but the wall time (and the BLAS rounding order, ~1e-16).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle

NEAR = 1e-6          # blocks whose exclusive mass lies this close to 1 - thr are excluded
MAX_ERR = 2e-2       # attention tolerances for bf16 inputs (same bar for f32 and fp8 runs)
MEAN_ERR = 2e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _pool_map(fn, items):
    """fn over items on a thread pool with single-threaded BLAS in each call (the oracle's
    numpy work releases the GIL); results in item order."""
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    with threadpool_limits(1), ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


def oracle_probs(q, k, n=64, scale=None):
    """Oracle reduced-map probabilities P [B,H,nb,nb] of q, k [B,H,S,D] (any device)."""
    B, H, S, _ = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    sc = scale if scale is not None else 1.0 / np.sqrt(q.shape[-1])
    res = _pool_map(lambda bh: oracle.row_softmax(oracle.reduced_map(oracle.block_pool(f64(q[bh]), n),
                                                                     oracle.block_pool(f64(k[bh]), n), sc)), heads)
    return np.stack(res).reshape(B, H, S // n, S // n)


def masks_from_probs(P, thr, or_plane=None):
    """Oracle CDF selection of each row of P [B,H,nb,nb] -> (keep, E)."""
    B, H, nb, _ = P.shape
    res = _pool_map(lambda x: oracle.cdf_select(x, thr), [P[b, h] for b in range(B) for h in range(H)])
    keep = np.stack([r[0] for r in res]).reshape(B, H, nb, nb)
    E = np.stack([r[1] for r in res]).reshape(B, H, nb, nb)
    if or_plane is not None:
        keep = oracle.mask_or(keep, np.broadcast_to(or_plane, keep.shape))
    return keep, E


def oracle_masks(q, k, thr, n=64, or_plane=None, scale=None):
    """Oracle NABLA masks and exclusive masses of q, k [B,H,S,D] (any device)."""
    B, H, S, _ = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    res = _pool_map(lambda bh: oracle.nabla_mask(f64(q[bh]), f64(k[bh]), n, thr, scale)[:2], heads)
    keep = np.stack([r[0] for r in res]).reshape(B, H, S // n, S // n)
    E = np.stack([r[1] for r in res]).reshape(B, H, S // n, S // n)
    if or_plane is not None:
        keep = oracle.mask_or(keep, np.broadcast_to(or_plane, keep.shape))
    return keep, E


# Probabilities closer than this (relative) are equal up to the fp64 rounding of the reduced
# map: the GPU's and the oracle's maps sum the same products in different orders (a few
# ulps of |L| <= ~100 moves p by ~1e-14 relative), so either may order such entries first.
TIE_REL = 1e-12


def compare_masks(gpu_mask: torch.Tensor, keep: np.ndarray, E: np.ndarray, thr: float, P=None):
    """Bit-exact except entries within NEAR of the threshold; returns (#mismatch, #near).

    With the oracle's probabilities P, a row may also differ at its pivot by entries whose
    p agree with the pivot's (the smallest p the oracle's rule keeps) within TIE_REL: in
    either order the rule picks a valid prefix. Such entries are excused only when the
    row's excused differences balance (as many kept as dropped) and are printed."""
    g = gpu_mask.cpu().numpy().astype(bool)
    assert g.shape == keep.shape
    near = np.abs(E - (1.0 - thr)) <= NEAR
    bad = (g != keep) & ~near
    if P is not None and bad.any():
        rule = E < (1.0 - thr)                       # the oracle's selection before any OR
        for idx in zip(*np.nonzero(bad.any(axis=-1))):
            row_p, row_bad = P[idx], bad[idx]
            p_piv = row_p[rule[idx]].min()
            tie = np.abs(row_p - p_piv) <= TIE_REL * p_piv
            cand = row_bad & tie
            if cand.any() and (g[idx][cand].astype(int) - keep[idx][cand].astype(int)).sum() == 0:
                for j in np.nonzero(cand)[0]:
                    print(f"  excused tie at the pivot: row {idx} block {j} p {row_p[j]:.17g} "
                          f"(pivot p {p_piv:.17g})", flush=True)
                bad[idx] &= ~cand
    return int(bad.sum()), int(near.sum())


def oracle_attention_blocks(q, k, v, keep, blocks, s_valid, scale=None, q_deq=None, k_deq=None):
    """Oracle outputs for the listed (b, h, i) query blocks -> {(b,h,i): O [64, D]}.

    q_deq, k_deq: optional dequantised fp8 Q/K (per-head callables or [B,H,S,D] arrays)
    that the oracle consumes in place of q, k."""
    out = {}
    by_head = {}
    for (b, h, i) in blocks:
        by_head.setdefault((b, h), []).append(i)

    def get(x, b, h):
        return x(b, h) if callable(x) else x[b, h]

    for (b, h), idx in by_head.items():
        qq = get(q_deq, b, h) if q_deq is not None else f64(q[b, h])
        kk = get(k_deq, b, h) if k_deq is not None else f64(k[b, h])
        vv = f64(v[b, h])
        idx = sorted(set(idx))
        nt = _threads()
        chunks = [idx[c::nt] for c in range(min(nt, len(idx)))]
        res = _pool_map(lambda ch: oracle.block_sparse_attention(qq, kk, vv, keep[b, h], 64, s_valid, scale,
                                                                 q_blocks=ch)[0], chunks)
        for ch, O in zip(chunks, res):
            for i in ch:
                out[(b, h, i)] = O[i * 64:(i + 1) * 64]
    return out


def attention_errors(gpu_out: torch.Tensor, ref: dict):
    errs = []
    for (b, h, i), O in ref.items():
        g = f64(gpu_out[b, h, i * 64:(i + 1) * 64])
        errs.append(np.abs(g - O).ravel())
    e = np.concatenate(errs)
    return float(e.max()), float(e.mean())


def sample_blocks(keep: np.ndarray, per_head: int, seed: int = 0, full_heads=()):
    """(b, h, i) query blocks: all rows of `full_heads`, else `per_head` seeded rows per head
    that always include the first, last, densest and sparsest rows."""
    B, H, nb, _ = keep.shape
    rng = np.random.default_rng(seed)
    out = []
    counts = keep.sum(-1)
    for b in range(B):
        for h in range(H):
            if h in full_heads:
                out += [(b, h, i) for i in range(nb)]
                continue
            pick = {0, nb - 1, int(counts[b, h].argmax()), int(counts[b, h].argmin())}
            while len(pick) < min(per_head, nb):
                pick.add(int(rng.integers(nb)))
            out += [(b, h, i) for i in sorted(pick)]
    return out

# Gradient tolerances per head, relative to the largest reference gradient. Three
# roundings enter: P and dS as bf16 MFMA operands (unit roundoff 2^-8), the bf16 output,
# and delta = <dO, O> formed from the forward's bf16 output O. Since sum_k dS_qk = 0, dQ
# and dK are sums with cancellation, so these roundings are relative to the absolute
# terms, not to the result: each of the first and the last moves dQ by up to ~1% of
# max |dQ| on the 2B-DiT shape (fp64 emulation of the roundings), hence
# max |err| <= 4e-2 * max |ref|; the mean bound is the forward's, 2e-3 * max |ref|.
GRAD_MAX_REL = 4e-2
GRAD_MEAN_REL = 2e-3


def grad_errors(gpu: torch.Tensor, ref: np.ndarray, rows):
    """(max |err|, mean |err|, max |ref|) of gpu[rows] against ref[rows] ([S, D] per head)."""
    g = f64(gpu)[rows]
    r = ref[rows]
    assert np.isfinite(r).all()
    e = np.abs(g - r)
    return float(e.max()), float(e.mean()), float(np.abs(r).max())
