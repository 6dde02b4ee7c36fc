"""Shared helpers of the GPU parity tests: oracle reference values and comparisons."""
import numpy as np
import torch

import oracle

NEAR = 1e-6          # blocks whose exclusive mass lies this close to 1 - thr are excluded
MAX_ERR = 2e-2       # attention tolerances for bf16 inputs (same bar for f32 and fp8 runs)
MEAN_ERR = 2e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_masks(q, k, thr, n=64, or_plane=None):
    """Oracle NABLA masks and exclusive masses of q, k [B,H,S,D] (any device)."""
    B, H, S, _ = q.shape
    nb = S // n
    keep = np.zeros((B, H, nb, nb), dtype=bool)
    E = np.zeros((B, H, nb, nb))
    for b in range(B):
        for h in range(H):
            keep[b, h], E[b, h], _ = oracle.nabla_mask(f64(q[b, h]), f64(k[b, h]), n, thr)
    if or_plane is not None:
        keep = oracle.mask_or(keep, np.broadcast_to(or_plane, keep.shape))
    return keep, E


def compare_masks(gpu_mask: torch.Tensor, keep: np.ndarray, E: np.ndarray, thr: float):
    """Bit-exact except entries within NEAR of the threshold; returns (#mismatch, #near)."""
    g = gpu_mask.cpu().numpy().astype(bool)
    assert g.shape == keep.shape
    near = np.abs(E - (1.0 - thr)) <= NEAR
    bad = (g != keep) & ~near
    return int(bad.sum()), int(near.sum())


def oracle_attention_blocks(q, k, v, keep, blocks, s_valid, scale=None, q_deq=None, k_deq=None):
    """Oracle outputs for the listed (b, h, i) query blocks -> {(b,h,i): O [64, D]}."""
    out = {}
    by_head = {}
    for (b, h, i) in blocks:
        by_head.setdefault((b, h), []).append(i)
    for (b, h), idx in by_head.items():
        qq = q_deq[b, h] if q_deq is not None else f64(q[b, h])
        kk = k_deq[b, h] if k_deq is not None else f64(k[b, h])
        O, _ = oracle.block_sparse_attention(qq, kk, f64(v[b, h]), keep[b, h], 64, s_valid, scale,
                                             q_blocks=sorted(set(idx)))
        for i in idx:
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
# roundings enter: P and dS as bf16 MFMA operands (unit roundoff 2^-9), the bf16 output,
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
