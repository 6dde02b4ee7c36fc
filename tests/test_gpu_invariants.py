"""Invariants that the pages and the mathematics fix, re-checked on the GPU's own outputs.

Beside the element-wise parity tests, these hold for any correct implementation and catch
mistakes that a comparison at a few thresholds could miss:
  * NABLA (review, "Core claim"): the kept set of each row covers reduced mass >= 1 - thr
    (measured with the oracle's probabilities; blocks the library flags as near the
    threshold are the only ones allowed to decide it differently), and the kept set grows as
    thr falls, exactly, since both are decided on the same fixed-point masses;
  * every row keeps its top block, no dropped block outweighs a kept one, and permuting
    whole blocks of Q and K permutes the mask alike;
  * Top-k: exactly min(k, nb) blocks per row;
  * attention (online softmax, FlashAttention abstract): every output row lies in the box
    spanned by the V rows it may attend to (a convex combination, up to the bf16 rounding
    of the output), rows with nothing allowed are 0, and lse is finite exactly there.
"""
import numpy as np
import pytest
import torch

from synth import get_config, make_inputs
from parity_util import f64, oracle_probs

pytestmark = pytest.mark.gpu
DEV = "cuda"
THRS = (0.0, 0.05, 0.1, 0.2, 0.4, 0.7, 0.95)


@pytest.mark.parametrize("cid,heads", [(2, 4), (3, 2)])   # short rows (nb 128) and long rows (nb 1182)
def test_mask_monotone_in_thr_and_covers_mass(gpu_lib, cid, heads):
    cfg = get_config(cid, heads=heads)
    q, k, _ = make_inputs(cfg, seed=11, device=DEV)
    P = oracle_probs(q, k)
    prev = None
    for thr in THRS:
        mask, near = gpu_lib.nabla_build_mask(q, k, thr, near=True)
        torch.cuda.synchronize()
        m = mask.cpu().numpy().astype(bool)
        nr = near.cpu().numpy().astype(bool)
        # coverage: the kept mass reaches 1 - thr, up to the mass of flagged blocks
        kept_mass = (P * m).sum(axis=-1)
        slack = (P * (nr & ~m)).sum(axis=-1)
        assert np.all(kept_mass + slack >= (1.0 - thr) - 1e-9), thr
        # minimality: dropping the smallest kept unflagged block falls below 1 - thr
        for idx in np.ndindex(m.shape[:-1]):
            row, p, fl = m[idx], P[idx], nr[idx]
            if row.sum() > 1:
                j = np.flatnonzero(row)[np.argmin(p[row])]
                if not fl[j]:
                    assert kept_mass[idx] - p[j] < (1.0 - thr) + 1e-9, (thr, idx)
        if prev is not None:
            assert np.all(prev | ~m), thr      # kept at this thr => kept at every smaller thr
        prev = m
    print(f"[invariants] masks at {len(THRS)} thresholds: monotone, covering", flush=True)


def test_topk_counts(gpu_lib):
    cfg = get_config(2, heads=3)
    q, k, _ = make_inputs(cfg, seed=12, device=DEV)
    for topk in (1, 7, 64, cfg.nb, cfg.nb + 5):
        m = gpu_lib.nabla_build_mask_topk(q, k, topk)
        torch.cuda.synchronize()
        assert torch.all(m.sum(dim=-1) == min(topk, cfg.nb)), topk


@pytest.mark.parametrize("cid,heads", [(2, 4), (3, 2)])
def test_attention_rows_are_convex_combinations(gpu_lib, cid, heads):
    cfg = get_config(cid, heads=heads)
    q, k, v = make_inputs(cfg, seed=13, device=DEV)
    thr = cfg.thrs[0] if cfg.thrs else 0.2
    mask = gpu_lib.nabla_build_mask(q, k, thr)
    mask[:, :, 3] = 0                         # a row with nothing allowed
    out, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, s_valid=cfg.S_valid, return_lse=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().astype(bool)
    nb, S = cfg.nb, cfg.S
    rng = np.random.default_rng(cid)
    blocks = sorted(set([0, 3, nb - 1] + rng.integers(0, nb, 12).tolist()))
    for h in range(cfg.H):
        vh = f64(v[0, h])
        o = f64(out[0, h])
        L = lse[0, h].cpu().numpy()
        for i in blocks:
            cols = np.concatenate([np.arange(j * 64, (j + 1) * 64) for j in np.flatnonzero(m[0, h, i])]) \
                if m[0, h, i].any() else np.zeros(0, dtype=np.int64)
            cols = cols[cols < cfg.S_valid]
            rows = np.arange(i * 64, min((i + 1) * 64, S))
            valid = rows < cfg.S_valid
            if len(cols) == 0:
                assert np.all(o[rows] == 0) and np.all(np.isneginf(L[rows]))
                continue
            lo, hi = vh[cols].min(axis=0), vh[cols].max(axis=0)
            tol = 2.0 ** -8 * np.maximum(np.abs(lo), np.abs(hi)) + 1e-6   # bf16 rounding of the output
            r = rows[valid]
            assert np.all(o[r] >= lo - tol) and np.all(o[r] <= hi + tol), (h, i)
            assert np.all(np.isfinite(L[r])) and np.all(np.isneginf(L[rows[~valid]]))
            assert np.all(o[rows[~valid]] == 0)
    print(f"[invariants] {cfg.name}: {len(blocks)} blocks x {cfg.H} heads inside their V boxes", flush=True)


@pytest.mark.parametrize("cid,heads", [(2, 4), (3, 2)])
def test_mask_rows_nonempty_and_separated(gpu_lib, cid, heads):
    """Every row keeps its top block; no dropped block outweighs a kept one, up to flagged
    (near-threshold) blocks."""
    cfg = get_config(cid, heads=heads)
    q, k, _ = make_inputs(cfg, seed=14, device=DEV)
    P = oracle_probs(q, k)
    for thr in THRS:
        mask, near = gpu_lib.nabla_build_mask(q, k, thr, near=True)
        torch.cuda.synchronize()
        m = mask.cpu().numpy().astype(bool)
        nr = near.cpu().numpy().astype(bool)
        assert np.all(m.any(axis=-1)), thr
        for idx in np.ndindex(m.shape[:-1]):
            row, p, fl = m[idx], P[idx], nr[idx]
            kept, dropped = p[row & ~fl], p[~row & ~fl]
            if kept.size and dropped.size:   # entries equal to fp64 rounding may sort either way
                assert kept.min() >= dropped.max() * (1.0 - 1e-12), (thr, idx)


def test_mask_block_permutation_equivariance(gpu_lib):
    """Permuting whole 64-token blocks of Q (rows of the map) and of K (its columns) permutes
    the mask the same way, up to blocks flagged as near the threshold in either run (the
    row sums are taken in another order, so the last bits of the masses move)."""
    cfg = get_config(2, heads=3)
    q, k, _ = make_inputs(cfg, seed=15, device=DEV)
    nb = cfg.nb
    rng = np.random.default_rng(15)
    sq, sk = rng.permutation(nb), rng.permutation(nb)
    tok = lambda perm: torch.from_numpy(np.concatenate([np.arange(j * 64, (j + 1) * 64) for j in perm])).to(DEV)
    qp = q[:, :, tok(sq)].contiguous()
    kp = k[:, :, tok(sk)].contiguous()
    for thr in (0.05, 0.2, 0.6):
        m0, n0 = gpu_lib.nabla_build_mask(q, k, thr, near=True)
        m1, n1 = gpu_lib.nabla_build_mask(qp, kp, thr, near=True)
        torch.cuda.synchronize()
        a = m0.cpu().numpy().astype(bool)[:, :, sq][:, :, :, sk]
        fa = n0.cpu().numpy().astype(bool)[:, :, sq][:, :, :, sk]
        b = m1.cpu().numpy().astype(bool)
        fb = n1.cpu().numpy().astype(bool)
        diff = (a != b) & ~fa & ~fb
        assert not diff.any(), (thr, int(diff.sum()))
