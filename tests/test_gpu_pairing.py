"""GPU tests of the attention's pairing offsets (pairs of query blocks at a per-head offset d
chosen for alike kv lists, from nb = 512 on for shapes without a work order).

The chosen offsets are integers and are compared exactly with the argmin computed here
from the mask (union steps of every candidate pairing, ties to the smaller d). The
pairing only decides which two blocks share a workgroup; each block still walks its own
list in ascending order, so outputs must equal, bit for bit, those of the adjacent pairs
of the work-order path (the same heads run a few at a time), and every block is written.
"""
import numpy as np
import pytest
import torch

from parity_util import MAX_ERR, MEAN_ERR, attention_errors, oracle_attention_blocks

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair_blocks(p, d, nb):
    full = nb // (2 * d) * (2 * d)
    if 2 * p < full:
        r = p // d
        a = 2 * r * d + (p - r * d)
        return a, a + d
    a = full + 2 * (p - full // 2)
    return a, (a + 1 if a + 1 < nb else -1)


def _expected_offsets(keep):
    """argmin over d of sum over pairs |list(a) u list(b)|, ties to the smaller d."""
    B, H, nb, _ = keep.shape
    out = []
    for b in range(B):
        for h in range(H):
            m = keep[b, h]
            best = None
            for d in range(1, max(1, min(64, nb // 2)) + 1):
                xy = np.array([_pair_blocks(p, d, nb) for p in range((nb + 1) // 2)])
                two = xy[:, 1] >= 0
                c = int((m[xy[two, 0]] | m[xy[two, 1]]).sum()) + int(m[xy[~two, 0]].sum())
                if best is None or c < best[0]:
                    best = (c, d)
            out.append(best[1])
    return np.array(out)


def _structured_mask(H, nb, offsets, density, seed):
    """Head h: block i keeps the list of class i mod offsets[h] (so i and i + d agree),
    plus a few random extras and the diagonal."""
    rng = np.random.default_rng(seed)
    keep = np.zeros((1, H, nb, nb), bool)
    for h, d in enumerate(offsets):
        base = rng.random((d, nb)) < density
        keep[0, h] = base[np.arange(nb) % d]
        keep[0, h] |= rng.random((nb, nb)) < 0.01
        keep[0, h, np.arange(nb), np.arange(nb)] = True
    return keep


def test_pairing_offsets_match_argmin(gpu_lib):
    H, nb = 5, 600
    keep = _structured_mask(H, nb, [1, 55, 7, 64, 2], 0.15, 1)
    keep[0, 3] = False                  # an empty head: every d costs 0, d = 1 is chosen
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    q = torch.empty(1, H, nb * 64, 128, dtype=torch.bfloat16, device=DEV)
    rp, ci = gpu_lib.mask_to_csr(mask)
    got = gpu_lib.attn_pair_offsets(q, rp, ci).cpu().numpy()
    want = _expected_offsets(keep)
    print(f"[pairing] offsets {got.tolist()} expected {want.tolist()}", flush=True)
    assert np.array_equal(got, want)
    assert want[1] == 55 and want[3] == 1
    # the same from fixed-stride lists (stride nb)
    rows = H * nb
    rp_h = rp.cpu().numpy()
    kv_len = torch.from_numpy(np.diff(rp_h).astype(np.int32)).to(DEV)
    kv_idx = torch.zeros(rows * nb, dtype=torch.int32)
    ci_h = ci.cpu()
    for r in range(rows):
        kv_idx[r * nb: r * nb + rp_h[r + 1] - rp_h[r]] = ci_h[rp_h[r]:rp_h[r + 1]]
    got2 = gpu_lib.attn_pair_offsets(q, None, kv_idx.to(DEV), kv_len=kv_len).cpu().numpy()
    assert np.array_equal(got2, want)


@pytest.mark.parametrize("nb", [512, 515])
def test_pairing_outputs_equal_adjacent_pairs(gpu_lib, nb):
    """16 heads of 512 (515: odd, ragged last runs) blocks run with pairing offsets. At 512,
    2 heads at a time run in the work order with adjacent pairs, and the results are equal
    bit for bit; every block is written (NaN-initialised output) and sampled blocks are
    within the oracle tolerance."""
    H, D = 16, 128
    S = nb * 64
    sv = S - 23
    offsets = [1, 55, 3, 64, 9, 2, 40, 1, 17, 33, 5, 56, 1, 12, 63, 8]
    keep = _structured_mask(H, nb, offsets, 0.1, nb)
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    g = torch.Generator(device="cpu").manual_seed(nb)
    q, k, v = (torch.randn(1, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    assert gpu_lib.attn_work_order_slots(q, sv) == 0           # the pairing path
    adjacent = gpu_lib.attn_work_order_slots(q[:, :2], sv) > 0 # 2 heads: adjacent pairs in the work order
    assert adjacent == (nb <= 512)
    rp, ci = gpu_lib.mask_to_csr(mask)
    print(f"[pairing] nb {nb}: offsets {gpu_lib.attn_pair_offsets(q, rp, ci, s_valid=sv).tolist()}", flush=True)
    out = torch.full_like(v, float("nan"))
    out, lse = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=sv, out=out, return_lse=True)
    out, lse = out.clone(), lse.clone()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for h0 in range(0, H if adjacent else 0, 2):
        sl = slice(h0, h0 + 2)
        qs, ks, vs = (t[:, sl].contiguous() for t in (q, k, v))
        o2, l2 = gpu_lib.block_sparse_attn_fwd(qs, ks, vs, mask[:, sl].contiguous(), s_valid=sv, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o2, out[:, sl]) and torch.equal(l2, lse[:, sl])
    blocks = [(0, h, i) for h in (1, 3, 14) for i in (0, 1, 54, 55, nb // 2, nb - 2, nb - 1)]
    mx, mean = attention_errors(out, oracle_attention_blocks(q, k, v, keep, blocks, sv))
    print(f"  max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


@pytest.mark.parametrize("heads", [3, 5])
def test_xcd_pair_placement_writes_every_block(gpu_lib, heads):
    """14B shape with an odd head count (items that do not split evenly over the XCD pairs):
    its heads pair blocks one frame apart, so pairs of XCDs share ranges and take their items
    alternately. Every valid output row is written (NaN-initialised output) and each head's
    output equals a single-head launch of it bit for bit."""
    from synth import get_config, make_inputs
    cfg = get_config(3, heads=heads)
    q, k, v = make_inputs(cfg, seed=4, device=DEV)
    m = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0])
    rp, ci = gpu_lib.mask_to_csr(m)
    d = gpu_lib.attn_pair_offsets(q, rp, ci, s_valid=cfg.S_valid)
    assert int(d[0]) > 1, "this shape should pair blocks at an offset above 1"
    out = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=cfg.S_valid, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :, :cfg.S_valid]).all()
    assert torch.all(out[:, :, cfg.S_valid:] == 0)
    for h in range(heads):
        sl = slice(h, h + 1)
        one = gpu_lib.block_sparse_attn_fwd(q[:, sl], k[:, sl], v[:, sl], m[:, sl], s_valid=cfg.S_valid)
        torch.cuda.synchronize()
        assert torch.equal(out[:, sl], one), h
