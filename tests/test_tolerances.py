"""Where the parity tolerances come from (CPU only).

The gradient bound GRAD_MAX_REL: the backward kernels round three quantities that the
plain derivative does not round -- the probabilities P and the score gradients dS become
bf16 MFMA operands, and delta = <dO, O> is formed from the forward's bf16 output O. An
fp64 emulation that inserts exactly these roundings (and nothing else) measures the
error they cause on a 2B-DiT-like head; the tolerance must exceed it with a margin of 3
for the fp32 accumulation order and the final output rounding, which the emulation
leaves out. Also: compare_masks excuses a pivot tie only when the difference is a swap
of entries whose probabilities agree to the map's fp64 rounding; and the lse bound: the
attention normalises by the fp32 sum of its probabilities as rounded to bf16, so lse lies
within -log(1 - 2^-8) of exact (bf16 keeps 8 significant bits).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from parity_util import GRAD_MAX_REL, TIE_REL, compare_masks


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def _dq_rows(q, k, v, do, keep, rows_of, s_valid, scale, round_ops):
    """dQ of the query blocks in rows_of, with (round_ops) or without the kernels' bf16
    roundings of P, dS and the O used for delta."""
    out = {}
    n = 64
    for i in rows_of:
        rows = np.arange(i * n, min((i + 1) * n, s_valid))
        kept = np.nonzero(keep[i])[0]
        cols = np.concatenate([np.arange(j * n, (j + 1) * n) for j in kept])
        cols = cols[cols < s_valid]
        s = scale * (q[rows] @ k[cols].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        P = e / e.sum(axis=1, keepdims=True)
        O = P @ v[cols]
        dP = do[rows] @ v[cols].T
        delta = (do[rows] * (_bf16(O) if round_ops else O)).sum(axis=1, keepdims=True)
        dS = P * (dP - delta)
        if round_ops:
            dS = _bf16(dS)
        out[i] = scale * (dS @ k[cols])
    return out


def test_gradient_tolerance_covers_the_prescribed_roundings():
    cfg = get_config(2, heads=1)
    q, k, v = (x[0, 0].double().numpy() for x in make_inputs(cfg, seed=0))
    do = np.random.default_rng(3).standard_normal(q.shape)
    do = _bf16(do)
    plane = oracle.sta_block_mask(cfg.grid, cfg.order, cfg.order_tile, cfg.sta.tile, cfg.sta.window, 64, cfg.S)
    keep, _, _ = oracle.nabla_mask(q, k, 64, cfg.thrs[0])
    keep |= plane
    scale = 1.0 / np.sqrt(cfg.D)
    blocks = list(range(0, cfg.nb, 4))
    exact = _dq_rows(q, k, v, do, keep, blocks, cfg.S_valid, scale, False)
    rounded = _dq_rows(q, k, v, do, keep, blocks, cfg.S_valid, scale, True)
    ref_max = max(np.abs(x).max() for x in exact.values())
    err = max(np.abs(rounded[i] - exact[i]).max() for i in blocks)
    rel = err / ref_max
    print(f"emulated bf16 P/dS/O roundings: max |err| = {rel:.4f} of max |dQ|")
    # the roundings alone cost about 1% of max |dQ| here (sums with cancellation: the
    # errors are relative to the terms, not to the result) ...
    assert 0.003 < rel
    # ... and the tolerance leaves a factor of 3 above them
    assert 3 * rel <= GRAD_MAX_REL


def test_compare_masks_excuses_only_pivot_ties():
    # one row, oracle order 0 > 1 = 2 (tie to 1e-15 relative) > 3; thr keeps two entries
    p = np.array([[0.5, 0.2, 0.2 * (1 + 1e-15), 0.1]])
    p = p / p.sum()
    keep, E = oracle.cdf_select(p, 0.35)
    assert keep.sum() == 2
    P4, keep4, E4 = p[None, None], keep[None, None], E[None, None]
    swapped = keep.copy()
    j_kept = [j for j in (1, 2) if keep[0, j]][0]
    j_drop = 3 - j_kept
    swapped[0, j_kept], swapped[0, j_drop] = False, True
    g = torch.from_numpy(swapped[None, None].astype(np.uint8))
    assert compare_masks(g, keep4, E4, 0.35)[0] == 2                 # strict without P
    assert compare_masks(g, keep4, E4, 0.35, P=P4)[0] == 0           # a tie at the pivot
    # a swap with an entry that is not tied is never excused
    wrong = keep.copy()
    wrong[0, j_kept], wrong[0, 3] = False, True
    assert compare_masks(torch.from_numpy(wrong[None, None].astype(np.uint8)), keep4, E4, 0.35, P=P4)[0] == 2
    # an extra kept tied entry (unbalanced) is not excused either
    extra = keep.copy()
    extra[0, j_drop] = True
    assert compare_masks(torch.from_numpy(extra[None, None].astype(np.uint8)), keep4, E4, 0.35, P=P4)[0] == 1
    assert TIE_REL < 1e-9


def test_lse_bound_of_the_bf16_normaliser():
    """Each probability rounded to bf16 (round to nearest even, 8 significant bits) is within
    2^-8 (relative) of exact, so the sum of the rounded terms is within that factor of the
    exact sum and lse within -log(1 - 2^-8) ~ 3.9e-3. Terms all just below a rounding
    midpoint (1 + 2^-8 - 2^-20 rounds to 1) come within 0.5% of the bound, so a bound from a
    unit roundoff of 2^-9 would be wrong; rows of random scores under the kernel's offsets
    (the running maximum, or up to 8 below the row maximum with the lazy rescale) stay inside."""
    bound = -np.log1p(-2.0 ** -8)
    x = np.full(1000, 1.0 + 2.0 ** -8 - 2.0 ** -20)
    worst = abs(np.log(_bf16(x).sum()) - np.log(x.sum()))
    assert 0.995 * bound < worst <= bound
    assert worst > -np.log1p(-2.0 ** -9)
    rng = np.random.default_rng(3)
    for sigma in (0.5, 3.0, 12.0):
        s = rng.normal(0.0, sigma, (200, 512))
        for shift in (0.0, 4.0, 8.0):
            m = s.max(axis=1, keepdims=True) - shift
            p = np.exp2(s - m)
            err = np.abs(np.log(_bf16(p).sum(axis=1)) - np.log(p.sum(axis=1)))
            assert err.max() <= bound, (sigma, shift, err.max())
