"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Masks are compared bit for bit, except blocks whose exclusive cumulative mass lies
within 1e-6 of 1 - thr (counted and printed). Attention is compared with the oracle's
mask, max |err| <= 2e-2 and mean |err| <= 2e-3, on every query block where the oracle
is cheap and on seeded samples (always with the first, last, densest and sparsest rows)
at the full workload sizes.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs, quantize_fp8_blocks
from parity_util import (MAX_ERR, MEAN_ERR, NEAR, attention_errors, compare_masks, f64, oracle_attention_blocks,
                         oracle_masks, sample_blocks)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sta_plane(cfg):
    if cfg.sta is None:
        return None
    return oracle.sta_block_mask(cfg.grid, cfg.order, cfg.order_tile, cfg.sta.tile, cfg.sta.window, 64, cfg.S)


def _gpu_sta(bsa, cfg):
    return bsa.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                              order_tile=cfg.order_tile, device=DEV)


# ----------------------------------------------------------------------------- masks
@pytest.mark.parametrize("cid,heads", [(1, None), (2, None), (3, 40)])
def test_nabla_mask_parity(gpu_lib, cid, heads):
    cfg = get_config(cid, heads)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    for thr in cfg.thrs:
        print(f"[mask] config {cid} thr {thr} shape {tuple(q.shape)}", flush=True)
        m = gpu_lib.nabla_build_mask(q, k, thr)
        torch.cuda.synchronize()
        keep, E = oracle_masks(q, k, thr)
        bad, near = compare_masks(m, keep, E, thr)
        print(f"  mismatches {bad}, near-threshold entries {near}, kept {keep.mean():.4f}", flush=True)
        assert bad == 0


def test_nabla_mask_sweep_with_sta_or(gpu_lib):
    cfg = get_config(5, heads=6)
    q, k, v = make_inputs(cfg, seed=1, device=DEV)
    plane = _sta_plane(cfg)
    sta = _gpu_sta(gpu_lib, cfg)
    for thr in cfg.thrs:
        m = gpu_lib.nabla_build_mask(q, k, thr, or_mask=sta)
        torch.cuda.synchronize()
        keep, E = oracle_masks(q, k, thr, or_plane=plane)
        bad, near = compare_masks(m, keep, E, thr)
        print(f"[mask] config 5 thr {thr}: mismatches {bad}, near {near}, kept {keep.mean():.4f}", flush=True)
        assert bad == 0


def test_nabla_degenerate_rows(gpu_lib):
    """All-equal rows (q = 0): every key block ties; ties go by ascending index."""
    B, H, S, D = 1, 3, 64 * 37, 128
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(B, H, S, D, device=DEV).to(torch.bfloat16)
    for thr in (0.0, 0.3, 0.5, 0.99):
        m = gpu_lib.nabla_build_mask(q, k, thr)
        keep, E = oracle_masks(q, k, thr)
        bad, near = compare_masks(m, keep, E, thr)
        assert bad == 0, (thr, bad)


def test_nabla_thr_edges_and_determinism(gpu_lib):
    cfg = get_config(2, heads=4)
    q, k, _ = make_inputs(cfg, seed=3, device=DEV)
    for thr in (0.0, 0.999):
        m = gpu_lib.nabla_build_mask(q, k, thr)
        keep, E = oracle_masks(q, k, thr)
        assert compare_masks(m, keep, E, thr)[0] == 0
    a = gpu_lib.nabla_build_mask(q, k, 0.1).clone()
    b = gpu_lib.nabla_build_mask(q, k, 0.1)
    assert torch.equal(a, b)


def test_nabla_f32_and_d64(gpu_lib):
    cfg = get_config(1)
    q, k, _ = make_inputs(cfg, seed=4, device=DEV)
    # a longer f32 sequence with a ragged number of 16-row groups
    q2 = torch.randn(2, 2, 64 * 21, 64, device=DEV)
    k2 = torch.randn(2, 2, 64 * 21, 64, device=DEV)
    for (qq, kk) in ((q, k), (q2, k2), (q2.to(torch.bfloat16), k2.to(torch.bfloat16))):
        m = gpu_lib.nabla_build_mask(qq, kk, 0.2)
        keep, E = oracle_masks(qq, kk, 0.2)
        assert compare_masks(m, keep, E, 0.2)[0] == 0


# ----------------------------------------------------------------------------- STA / OR / CSR
@pytest.mark.parametrize("cid", [2, 4, 5])
def test_sta_mask_parity(gpu_lib, cid):
    cfg = get_config(cid)
    g = _gpu_sta(gpu_lib, cfg).cpu().numpy().astype(bool)
    assert np.array_equal(g, _sta_plane(cfg))


@pytest.mark.parametrize("grid,order,otile,tile,window", [
    ((3, 5, 7), "row", None, (2, 2, 3), (3, 3, 3)),
    ((5, 6, 7), "tile", (2, 4, 4), (2, 4, 4), (1, 3, 5)),
    ((4, 9, 10), "tile", (3, 4, 4), (2, 3, 5), (3, 1, 3)),
    # blocks aligned with the tiles (one and two blocks per tile): the single-kernel path
    ((4, 16, 16), "tile", (2, 8, 4), (2, 8, 4), (1, 3, 5)),
    ((6, 16, 24), "tile", (2, 8, 8), (2, 8, 8), (3, 3, 1)),
])
def test_sta_ragged_geometries(gpu_lib, grid, order, otile, tile, window):
    Sv = int(np.prod(grid))
    S = -(-Sv // 64) * 64
    g = gpu_lib.sta_build_mask(S, Sv, grid, tile, window, order=order, order_tile=otile, device=DEV)
    ref = oracle.sta_block_mask(grid, order, otile, tile, window, 64, S)
    assert np.array_equal(g.cpu().numpy().astype(bool), ref)


@pytest.mark.parametrize("cid,heads,thr", [(2, None, 0.1), (4, 2, 0.3), (5, 3, 0.2)])
def test_nabla_sta_one_call(gpu_lib, cid, heads, thr):
    """nabla_build_mask_sta equals nabla_build_mask OR'd with the sta_build_mask plane, bit
    for bit: aligned tile-major layouts (configs 2 and 4: the rule inside the short-row and
    the wide select) and a padded row-major one (config 5: the plane built first)."""
    cfg = get_config(cid, heads)
    q, k, _ = make_inputs(cfg, seed=0, device=DEV)
    plane = _gpu_sta(gpu_lib, cfg)
    ref = gpu_lib.nabla_build_mask(q, k, thr, or_mask=plane)
    one = gpu_lib.nabla_build_mask_sta(q, k, thr, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                       order_tile=cfg.order_tile, s_valid=cfg.S_valid)
    torch.cuda.synchronize()
    print(f"[nabla+sta] config {cid} nb {cfg.nb} kept {ref.float().mean().item():.4f}", flush=True)
    assert torch.equal(ref, one)


def test_mask_or_and_csr(gpu_lib):
    rng = np.random.default_rng(0)
    a = rng.random((2, 3, 37, 37)) < 0.2
    bplane = rng.random((37, 37)) < 0.3
    a[0, 1, 5] = False
    ta = torch.from_numpy(a.astype(np.uint8)).to(DEV)
    tb = torch.from_numpy(bplane.astype(np.uint8)).to(DEV)
    u = gpu_lib.mask_or(ta, tb)
    ref = oracle.mask_or(a, np.broadcast_to(bplane, a.shape))
    assert np.array_equal(u.cpu().numpy().astype(bool), ref)
    z = torch.zeros_like(ta)
    z[0, 1] = 1
    rp, ci, order = gpu_lib.mask_to_csr(ta, return_order=True)
    rp_ref, ci_ref = oracle.mask_to_csr(a.reshape(-1, 37))
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    assert np.array_equal(ci.cpu().numpy()[:rp_ref[-1]], ci_ref)
    assert np.array_equal(order.cpu().numpy(), oracle.longest_first_order(a.reshape(-1, 37)))


# ----------------------------------------------------------------------------- attention
def _attn_check(gpu_lib, cfg, q, k, v, keep, blocks, **kw):
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    out = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, s_valid=cfg.S_valid, **{x: y for x, y in kw.items()
                                                                                if x in ("q_scale", "k_scale")})
    torch.cuda.synchronize()
    ref = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid, q_deq=kw.get("q_deq"), k_deq=kw.get("k_deq"))
    mx, mean = attention_errors(out, ref)
    print(f"[attn] {cfg.name}: {len(blocks)} query blocks, max err {mx:.3e}, mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR
    return out


def test_attention_config1_f32_full(gpu_lib):
    cfg = get_config(1)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    keep, _ = oracle_masks(q, k, 0.2)
    blocks = [(0, h, i) for h in range(cfg.H) for i in range(cfg.nb)]
    _attn_check(gpu_lib, cfg, q, k, v, keep, blocks)
    # the same data in bf16 with head_dim 64
    _attn_check(gpu_lib, cfg, q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), keep, blocks)


def test_attention_config2_full(gpu_lib):
    cfg = get_config(2)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    keep, _ = oracle_masks(q, k, 0.1, or_plane=_sta_plane(cfg))
    blocks = [(0, h, i) for h in range(cfg.H) for i in range(cfg.nb)]
    _attn_check(gpu_lib, cfg, q, k, v, keep, blocks)


# The benchmarked workloads at full size (every head with its real mask, the bench's
# call path) are in test_gpu_workloads.py.


@pytest.mark.parametrize("mode,D,nb", [("fp8", 64, 2736), ("bf16", 64, 4100), ("bf16", 128, 8200)])
def test_attention_order_tables_past_shared_memory(gpu_lib, mode, D, nb):
    """One head with more key blocks than the in-kernel longest-first order can tabulate in
    the kernel's shared buffer (nb + 1 + ceil(nb/2) + 3 ints: past 4096 ints for fp8 D=64,
    6144 for bf16 D=64, 12288 for bf16 D=128): the workgroups keep the natural order, and
    every query block is still written (NaN-initialised output, every valid row finite);
    sampled blocks match the oracle."""
    B, H, S = 1, 1, nb * 64
    sv = S - 40
    g = torch.Generator(device="cpu").manual_seed(nb)
    q, k, v = (torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    rng = np.random.default_rng(nb)
    keep = np.zeros((B, H, nb, nb), bool)
    keep[0, 0, np.arange(nb), np.arange(nb)] = True
    keep[0, 0, np.arange(nb)[:, None], rng.integers(0, nb, size=(nb, 6))] = True
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    qs = ks = None
    qa, ka = q, k
    if mode == "fp8":
        qa, qs = gpu_lib.quantize_fp8_blocks(q)
        ka, ks = gpu_lib.quantize_fp8_blocks(k)
    rp, ci = gpu_lib.mask_to_csr(mask)
    print(f"[order tables] {mode} D {D} nb {nb}: slots {gpu_lib.attn_work_order_slots(q, sv)}", flush=True)
    out = torch.full_like(v, float("nan"))
    gpu_lib.block_sparse_attn_fwd_csr(qa, ka, v, rp, ci, s_valid=sv, q_scale=qs, k_scale=ks, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :, :sv]).all()
    blocks = [(0, 0, i) for i in (0, 1, nb // 3, nb // 2, nb - 2, nb - 1)]
    kw = {}
    if mode == "fp8":
        deq = lambda c, s: (c[0, 0].view(torch.float8_e4m3fn).double().view(nb, 64, D)
                            * s[0, 0].double()[:, None, None]).view(S, D).cpu().numpy()
        kw = dict(q_deq=lambda b, h: deq(qa, qs), k_deq=lambda b, h: deq(ka, ks))
    mx, mean = attention_errors(out, oracle_attention_blocks(q, k, v, keep, blocks, sv, **kw))
    print(f"  max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


def test_attention_edge_rows(gpu_lib):
    """Empty kv lists give zeros; a fully masked padding tail; D=64 and D=128."""
    for D in (64, 128):
        B, H, S, Sv = 1, 2, 64 * 6, 64 * 5 + 7
        q = torch.randn(B, H, S, D, device=DEV).to(torch.bfloat16)
        k = torch.randn(B, H, S, D, device=DEV).to(torch.bfloat16)
        v = torch.randn(B, H, S, D, device=DEV).to(torch.bfloat16)
        keep = np.random.default_rng(D).random((B, H, 6, 6)) < 0.5
        keep[0, 0, 2] = False              # a row with no kept block
        keep[0, 1, 3] = False
        keep[0, 1, 3, 5] = True            # only the partly padded last block
        mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
        out, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, s_valid=Sv, return_lse=True)
        torch.cuda.synchronize()
        assert torch.all(out[0, 0, 128:192] == 0)
        assert torch.all(out[:, :, Sv:] == 0)
        assert torch.isinf(lse[0, 0, 128:192]).all()
        for h in range(H):
            O, L = oracle.block_sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), keep[0, h], 64, Sv)
            assert np.abs(f64(out[0, h]) - O).max() <= MAX_ERR
            fin = np.isfinite(L)
            # lse is the log of the normaliser the kernel divides by: the sum of the weights
            # as rounded to bf16 for the PV product, each within 2^-8 (relative; bf16 has 8
            # significant bits) of exact, so |lse - exact| <= -log(1 - 2^-8) ~ 3.9e-3 in the
            # worst case (all roundings one way); the test holds it to 2.5e-3, inside that bound
            assert np.abs(f64(lse[0, h])[fin] - L[fin]).max() < 2.5e-3


def test_attention_determinism_and_csr_entry(gpu_lib):
    cfg = get_config(2, heads=4)
    q, k, v = make_inputs(cfg, seed=5, device=DEV)
    mask = gpu_lib.nabla_build_mask(q, k, 0.1)
    a = gpu_lib.block_sparse_attn_fwd(q, k, v, mask).clone()
    b = gpu_lib.block_sparse_attn_fwd(q, k, v, mask).clone()
    assert torch.equal(a, b)
    rp, ci = gpu_lib.mask_to_csr(mask)
    c = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci)
    assert torch.equal(a, c)


def test_full_mask_equals_dense(gpu_lib):
    cfg = get_config(2, heads=2)
    q, k, v = make_inputs(cfg, seed=6, device=DEV)
    ones = torch.ones(cfg.nb, cfg.nb, dtype=torch.uint8, device=DEV)
    out = gpu_lib.block_sparse_attn_fwd(q, k, v, ones)
    torch.cuda.synchronize()
    ref = torch.nn.functional.scaled_dot_product_attention(q.cpu().double(), k.cpu().double(), v.cpu().double())
    err = (out.cpu().double() - ref).abs()
    assert err.max().item() <= MAX_ERR and err.mean().item() <= MEAN_ERR


def test_attention_f32_d128(gpu_lib):
    """f32 inputs with head_dim 128 (hi/lo bf16 split path) on a ragged sequence."""
    B, H, S, Sv, D = 1, 2, 64 * 5, 64 * 4 + 9, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    q, k, v = (torch.randn(B, H, S, D, device=DEV, generator=g) for _ in range(3))
    keep = np.random.default_rng(12).random((B, H, 5, 5)) < 0.6
    keep[:, :, np.arange(5), np.arange(5)] = True
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    out = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, s_valid=Sv)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    for h in range(H):
        O, _ = oracle.block_sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), keep[0, h], 64, Sv)
        err = np.abs(f64(out[0, h]) - O)
        assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR


def test_csr_multi_segment(gpu_lib):
    """More rows than one scan segment (1024), a broadcast plane, and empty rows."""
    rng = np.random.default_rng(21)
    m = rng.random((2, 9, 70, 70)) < 0.15
    m[1, 4, :10] = False
    t = torch.from_numpy(m.astype(np.uint8)).to(DEV)
    rp, ci, order = gpu_lib.mask_to_csr(t, return_order=True)
    rp_ref, ci_ref = oracle.mask_to_csr(m.reshape(-1, 70))
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    assert np.array_equal(ci.cpu().numpy()[:rp_ref[-1]], ci_ref)
    assert np.array_equal(order.cpu().numpy(), oracle.longest_first_order(m.reshape(-1, 70)))
    plane = torch.from_numpy(m[0, 0].astype(np.uint8)).to(DEV)
    rp2, ci2, order2 = gpu_lib.mask_to_csr(plane, B=2, H=9, return_order=True)
    m2 = np.broadcast_to(m[0, 0], (18, 70, 70)).reshape(-1, 70)
    rp2_ref, ci2_ref = oracle.mask_to_csr(m2)
    assert np.array_equal(rp2.cpu().numpy(), rp2_ref)
    assert np.array_equal(ci2.cpu().numpy()[:rp2_ref[-1]], ci2_ref)
    assert np.array_equal(order2.cpu().numpy(), oracle.longest_first_order(m2))


def test_csr_small_single_launch(gpu_lib):
    """Masks small enough for the one-workgroup builder (nb a multiple of 16): empty and
    full rows, nonzero values other than 1, a broadcast plane, and the largest size."""
    rng = np.random.default_rng(33)
    m = (rng.random((2, 3, 96, 96)) < 0.3).astype(np.uint8) * rng.integers(1, 255, (2, 3, 96, 96)).astype(np.uint8)
    m[0, 2, 7] = 0
    m[1, 0, 50] = 9
    t = torch.from_numpy(m).to(DEV)
    rp, ci = gpu_lib.mask_to_csr(t)
    rp_ref, ci_ref = oracle.mask_to_csr(m.reshape(-1, 96) != 0)
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    assert np.array_equal(ci.cpu().numpy()[:rp_ref[-1]], ci_ref)
    plane = torch.from_numpy(m[1, 1]).to(DEV)
    rp2, ci2 = gpu_lib.mask_to_csr(plane, B=1, H=5)
    m2 = np.broadcast_to(m[1, 1] != 0, (5, 96, 96)).reshape(-1, 96)
    rp2_ref, ci2_ref = oracle.mask_to_csr(m2)
    assert np.array_equal(rp2.cpu().numpy(), rp2_ref)
    assert np.array_equal(ci2.cpu().numpy()[:rp2_ref[-1]], ci2_ref)
    big = rng.random((1, 32, 128, 128)) < 0.4          # 4096 rows: the size limit
    tb = torch.from_numpy(big.astype(np.uint8)).to(DEV)
    rp3, ci3 = gpu_lib.mask_to_csr(tb)
    rp3_ref, ci3_ref = oracle.mask_to_csr(big.reshape(-1, 128))
    assert np.array_equal(rp3.cpu().numpy(), rp3_ref)
    assert np.array_equal(ci3.cpu().numpy()[:rp3_ref[-1]], ci3_ref)


def test_attention_work_order(gpu_lib):
    """The attention work order: every pair exactly once, XCD range x % 8 of slot x a
    contiguous run of pairs, each range by decreasing longer-list length; results
    identical with the order passed in, computed inside, and through the dense entry."""
    cfg = get_config(2)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    plane = _gpu_sta(gpu_lib, cfg)
    mask = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0], or_mask=plane)
    rp, ci = gpu_lib.mask_to_csr(mask)
    order = gpu_lib.attn_work_order(q, rp)
    assert order is not None
    o = order.cpu().numpy()
    counts = np.diff(rp.cpu().numpy())
    npair = cfg.nb // 2
    items = cfg.B * cfg.H * npair
    assert sorted(o[o >= 0].tolist()) == list(range(items))
    for x in range(8):
        rng_items = o[x::8]
        rng_items = rng_items[rng_items >= 0]
        assert np.all(np.diff(np.sort(rng_items)) == 1)            # a contiguous run
        bh, p = rng_items // npair, rng_items % npair
        key = np.maximum(counts[bh * cfg.nb + 2 * p], counts[bh * cfg.nb + 2 * p + 1])
        assert np.all(np.diff(key) <= 0)                            # longest first
    a = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, work_order=order)
    b = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci)
    c = gpu_lib.block_sparse_attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("heads", [16, 48])
def test_csr_with_work_order_one_call(gpu_lib, heads):
    """bsa_mask_to_csr_ordered: the same kv lists as bsa_mask_to_csr and the work order
    attn_work_order gives for them (per XCD range the same pairs with the same decreasing
    keys; equal keys may come in another order), identical attention results. 16 heads
    (2048 rows) take the single-launch path, 48 heads (6144 rows) the two-launch one."""
    cfg = get_config(2, heads=heads)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    plane = _gpu_sta(gpu_lib, cfg)
    mask = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0], or_mask=plane)
    rp, ci = gpu_lib.mask_to_csr(mask)
    ref = gpu_lib.attn_work_order(q, rp)
    assert ref is not None
    wo = torch.full_like(ref, -7)
    rp2, ci2 = gpu_lib.mask_to_csr(mask, work_order=wo)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2)
    n = int(rp[-1].item())
    assert torch.equal(ci[:n], ci2[:n])
    counts = np.diff(rp.cpu().numpy())
    npair = cfg.nb // 2
    o, r = wo.cpu().numpy(), ref.cpu().numpy()
    assert not (o == -7).any()
    for x in range(8):
        a, b = o[x::8], r[x::8]
        assert np.array_equal(a < 0, b < 0)
        a, b = a[a >= 0], b[b >= 0]
        assert sorted(a.tolist()) == sorted(b.tolist())
        ka = np.maximum(counts[(a // npair) * cfg.nb + 2 * (a % npair)], counts[(a // npair) * cfg.nb + 2 * (a % npair) + 1])
        kb = np.maximum(counts[(b // npair) * cfg.nb + 2 * (b % npair)], counts[(b // npair) * cfg.nb + 2 * (b % npair) + 1])
        assert np.array_equal(ka, kb)
    out_a = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp2, ci2, work_order=wo)
    out_b = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, work_order=ref)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)


def _check_order(wo, counts, nb, items):
    """A work order: every pair once, XCD range x % 8 a contiguous run of pairs by
    decreasing longer-list length."""
    o = wo.cpu().numpy()
    npair = (nb + 1) // 2
    assert sorted(o[o >= 0].tolist()) == list(range(items))
    for x in range(8):
        r = o[x::8]
        r = r[r >= 0]
        assert np.all(np.diff(np.sort(r)) == 1)
        bh, p = r // npair, r % npair
        cB = np.where(2 * p + 1 < nb, counts[np.minimum(bh * nb + 2 * p + 1, len(counts) - 1)], 0)
        key = np.maximum(counts[bh * nb + 2 * p], cB)
        assert np.all(np.diff(key) <= 0)


@pytest.mark.parametrize("case", ["cfg2", "cfg2x48", "nb200", "nb200-sta-plane"])
def test_mask_lists_one_call(gpu_lib, case):
    """nabla_build_mask_lists: the mask bit for bit as the oracle's (and as
    nabla_build_mask_sta), each row's kv list = its kept blocks in ascending order, the
    work order (built by the select's last workgroup) a valid longest-first order, and
    block_sparse_attn_fwd_lists identical to block_sparse_attn_fwd_csr on the same mask
    (with that order, and with the order each attention workgroup derives from the
    lengths)."""
    from dataclasses import replace
    sta_args = {}
    if case.startswith("cfg2"):
        cfg = get_config(2, heads=48 if case == "cfg2x48" else None)
        thr = 0.1
        sta_args = dict(grid=cfg.grid, tile=cfg.sta.tile, window=cfg.sta.window, order=cfg.order,
                        order_tile=cfg.order_tile)
        plane = _sta_plane(cfg)
    else:
        cfg = replace(get_config(3, heads=3), cid=9, name="short-8x40x40", grid=(8, 40, 40))
        thr = 0.2
        plane = None
        if case == "nb200-sta-plane":   # row-major, not aligned with the blocks: the plane path
            sta_args = dict(grid=cfg.grid, tile=(2, 8, 8), window=(3, 3, 3), order="row")
            plane = oracle.sta_block_mask(cfg.grid, "row", None, (2, 8, 8), (3, 3, 3), 64, cfg.S)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    nb, BH = cfg.nb, cfg.B * cfg.H
    print(f"[lists] {case}: heads {cfg.H} nb {nb} thr {thr} sta {bool(sta_args)}", flush=True)
    ws = gpu_lib.nabla_lists_workspace(q, cfg.S_valid)
    mask, kv_len, kv_idx, wo = gpu_lib.nabla_build_mask_lists(q, k, thr, s_valid=cfg.S_valid, ws=ws, **sta_args)
    torch.cuda.synchronize()
    keep, E = oracle_masks(q, k, thr, or_plane=plane)
    bad, near = compare_masks(mask, keep, E, thr)
    assert bad == 0, (bad, near)
    if sta_args:
        ref = gpu_lib.nabla_build_mask_sta(q, k, thr, s_valid=cfg.S_valid, **sta_args)
    else:
        ref = gpu_lib.nabla_build_mask(q, k, thr)
    torch.cuda.synchronize()
    assert torch.equal(mask, ref)
    m = mask.reshape(BH * nb, nb).cpu().numpy().astype(bool)
    counts = m.sum(1)
    assert np.array_equal(kv_len.cpu().numpy(), counts)
    idx = kv_idx.cpu().numpy()
    for r in range(BH * nb):
        assert np.array_equal(idx[r, :counts[r]], np.flatnonzero(m[r])), r
    assert wo is not None
    _check_order(wo, counts, nb, BH * ((nb + 1) // 2))
    # a second call on the same workspace (the arrival counter starts from zero again)
    mask2, kv_len2, kv_idx2, wo2 = gpu_lib.nabla_build_mask_lists(q, k, thr, s_valid=cfg.S_valid, ws=ws, **sta_args)
    torch.cuda.synchronize()
    assert torch.equal(mask2, mask) and torch.equal(kv_len2, kv_len)
    _check_order(wo2, counts, nb, BH * ((nb + 1) // 2))
    rp, ci = gpu_lib.mask_to_csr(mask)
    out_csr = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=cfg.S_valid)
    out_a = gpu_lib.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid, work_order=wo)
    out_b = gpu_lib.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_csr) and torch.equal(out_b, out_csr)
    blocks = sample_blocks(keep, 6, seed=3)
    refo = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid)
    mx, mean = attention_errors(out_a, refo)
    print(f"  {len(blocks)} query blocks: max err {mx:.3e}, mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mask_lists_ragged(gpu_lib, dtype):
    """The list path on an awkward shape: B = 2, 3 heads, nb = 37 (odd: the last pair has
    one block), S_valid = S - 40 with zero padding; bf16 and f32 (hi/lo split) inputs."""
    from dataclasses import replace
    cfg = replace(get_config(1), cid=9, name="ragged-37", B=2, H=3, grid=(1, 37, 64))
    assert cfg.nb == 37
    q, k, v = make_inputs(cfg, seed=5, device=DEV)
    sv = cfg.S - 40
    for t in (q, k, v):
        t[:, :, sv:] = 0
    q, k, v = (t.to(dtype) for t in (q, k, v))
    thr = 0.3
    mask, kv_len, kv_idx, wo = gpu_lib.nabla_build_mask_lists(q, k, thr, s_valid=sv)
    ref = gpu_lib.nabla_build_mask(q, k, thr)
    torch.cuda.synchronize()
    assert torch.equal(mask, ref)
    keep, E = oracle_masks(q, k, thr)
    bad, near = compare_masks(mask, keep, E, thr)
    assert bad == 0, (bad, near)
    BH, nb = cfg.B * cfg.H, cfg.nb
    m = mask.reshape(BH * nb, nb).cpu().numpy().astype(bool)
    counts = m.sum(1)
    assert np.array_equal(kv_len.cpu().numpy(), counts)
    idx = kv_idx.cpu().numpy()
    for r in range(BH * nb):
        assert np.array_equal(idx[r, :counts[r]], np.flatnonzero(m[r])), r
    assert wo is not None
    _check_order(wo, counts, nb, BH * ((nb + 1) // 2))
    rp, ci = gpu_lib.mask_to_csr(mask)
    out_csr = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=sv)
    out_l = gpu_lib.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=sv, work_order=wo)
    out_k = gpu_lib.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=sv)   # order derived in-kernel
    torch.cuda.synchronize()
    assert torch.equal(out_l, out_csr) and torch.equal(out_k, out_csr)
    blocks = [(b, h, i) for b in range(cfg.B) for h in range(cfg.H) for i in (0, 17, nb - 1)]
    refo = oracle_attention_blocks(q, k, v, keep, blocks, sv)
    mx, mean = attention_errors(out_l, refo)
    print(f"[lists ragged {dtype}] max err {mx:.3e}, mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


def test_longest_first_order_large(gpu_lib):
    """Several sort blocks and many equal counts (rows of a 40-head, nb=1182 mask with
    counts from a narrow band), and the largest nb the order supports in one head."""
    rng = np.random.default_rng(5)
    nb = 1182
    counts = rng.integers(380, 420, size=(40, nb))
    m = np.zeros((40, nb, nb), bool)
    for hh in range(40):
        for i in range(nb):
            m[hh, i, rng.choice(nb, counts[hh, i], replace=False)] = True
    t = torch.from_numpy(m.astype(np.uint8)).to(DEV).view(1, 40, nb, nb)
    rp, ci, order = gpu_lib.mask_to_csr(t, return_order=True)
    torch.cuda.synchronize()
    ref = oracle.longest_first_order(m.reshape(-1, nb))
    assert np.array_equal(order.cpu().numpy(), ref)
    nb2 = 16382
    plane = torch.zeros(nb2, nb2, dtype=torch.uint8, device=DEV)
    plane[:, :7] = 1
    plane[::3, 7:40] = 1
    rp, ci, order = gpu_lib.mask_to_csr(plane, B=1, H=1, return_order=True)
    ref = np.concatenate([np.arange(0, nb2, 3), np.setdiff1d(np.arange(nb2), np.arange(0, nb2, 3))])
    assert np.array_equal(order.cpu().numpy(), ref)


def test_maximum_nb_mask_topk_and_attention(gpu_lib):
    # nb = 2048 (the largest sequence the mask build accepts): the widest select instantiation
    from dataclasses import replace
    cfg = replace(get_config(3, heads=2), cid=9, name="max-32x64x64", grid=(32, 64, 64))
    assert cfg.nb == 2048 and cfg.S_valid == cfg.S
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    print(f"[max] nb {cfg.nb}, {cfg.H} heads", flush=True)
    m = gpu_lib.nabla_build_mask(q, k, 0.2)
    mt = gpu_lib.nabla_build_mask_topk(q, k, 300)
    torch.cuda.synchronize()
    keep, E = oracle_masks(q, k, 0.2)
    bad, near = compare_masks(m, keep, E, 0.2)
    print(f"  cdf mismatches {bad}, near {near}, kept {keep.mean():.4f}", flush=True)
    assert bad == 0
    for h in range(cfg.H):
        ref, _ = oracle.topk_mask(f64(q[0, h]), f64(k[0, h]), 64, 300)
        assert np.array_equal(mt[0, h].cpu().numpy().astype(bool), ref)
    out = gpu_lib.block_sparse_attn_fwd(q, k, v, m)
    torch.cuda.synchronize()
    blocks = [(0, h, i) for h in range(cfg.H) for i in (0, 1023, 2047)]
    mx, mean = attention_errors(out, oracle_attention_blocks(q, k, v, m.cpu().numpy().astype(bool), blocks, cfg.S))
    print(f"  attention max {mx:.3e} mean {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


@pytest.mark.parametrize("grid", [(3, 43, 64), (8, 40, 40), (16, 32, 32)])
def test_short_row_select_two_tiles(gpu_lib, grid):
    # nb = 129, 200, 256: the mask build for short rows (one wave per row once the map is
    # formed) with two column tiles per wave; thresholds, Top-k and an OR'd mask
    from dataclasses import replace
    cfg = replace(get_config(3, heads=3), cid=9, name="short-%dx%dx%d" % grid, grid=grid)
    assert cfg.S_valid == cfg.S and 128 < cfg.nb <= 256
    q, k, _ = make_inputs(cfg, seed=1, device=DEV)
    rng = np.random.default_rng(7)
    plane = rng.random((cfg.nb, cfg.nb)) < 0.05
    plane_t = torch.from_numpy(plane.astype(np.uint8)).to(DEV)
    for thr in (0.0, 0.1, 0.2, 0.6):
        print(f"[short] nb {cfg.nb} thr {thr}", flush=True)
        m = gpu_lib.nabla_build_mask(q, k, thr)
        mo = gpu_lib.nabla_build_mask(q, k, thr, or_mask=plane_t)
        torch.cuda.synchronize()
        keep, E = oracle_masks(q, k, thr)
        bad, near = compare_masks(m, keep, E, thr)
        assert bad == 0, (thr, bad, near)
        keep_or, _ = oracle_masks(q, k, thr, or_plane=plane)
        bad, near = compare_masks(mo, keep_or, E, thr)
        assert bad == 0, (thr, "or", bad, near)
    for topk in (1, 37, cfg.nb - 1):
        print(f"[short] nb {cfg.nb} topk {topk}", flush=True)
        mt = gpu_lib.nabla_build_mask_topk(q, k, topk)
        torch.cuda.synchronize()
        for h in range(cfg.H):
            ref, P = oracle.topk_mask(f64(q[0, h]), f64(k[0, h]), 64, topk)
            diff = mt[0, h].cpu().numpy().astype(bool) != ref
            kth = -np.sort(-P, axis=1)[:, topk - 1]
            assert not (diff & ~(np.abs(P - kth[:, None]) <= 2.0 ** -59)).any(), (topk, h)


def test_batched_model_layout_views(gpu_lib):
    """B = 2 with Q, K, V as [B, S, H, D] views of one packed QKV tensor (head and row strides of the
    model's layout, not contiguous [B, H, S, D]); the output written into a strided view too."""
    B, S, H, D, Sv = 2, 64 * 7, 3, 128, 64 * 6 + 20
    g = torch.Generator(device="cpu").manual_seed(21)
    qkv = torch.randn(B, S, 3, H, D, generator=g)
    pos = torch.sin(torch.arange(S)[:, None] * 0.05 + torch.arange(D)[None, :] * 0.3)   # some structure
    qkv[:, :, :2] += 2 * pos[None, :, None, None, :]
    qkv[:, Sv:] = 0
    qkv = qkv.to(torch.bfloat16).to(DEV)
    q, k, v = (qkv[:, :, t].permute(0, 2, 1, 3) for t in range(3))          # [B, H, S, D] views
    assert not q.is_contiguous() and q.stride(3) == 1
    m = gpu_lib.nabla_build_mask(q, k, 0.3)
    o2 = gpu_lib.block_sparse_attn_fwd(q, k, v, m, s_valid=Sv)
    obuf = torch.full((B, S, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    rp, ci = gpu_lib.mask_to_csr(m)
    gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=Sv, out=obuf.permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    assert torch.equal(obuf.permute(0, 2, 1, 3), o2)           # strided output, same values, every row written
    keep, E = oracle_masks(q, k, 0.3)
    bad, near = compare_masks(m, keep, E, 0.3)
    assert bad == 0
    for b in range(B):
        for h in range(H):
            O, _ = oracle.block_sparse_attention(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), keep[b, h], 64, Sv)
            err = np.abs(f64(o2[b, h]) - O)
            assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR, (b, h, err.max())


def test_attention_head_order_writes_every_block(gpu_lib):
    """Many rounds of long rows (nb = 512, 16 heads: more pairs than the ordered schedule
    takes): each attention workgroup derives its pair from the kv-list lengths, longest
    first inside each head. Every query block must be written exactly by its pair: the
    output starts as NaN and every valid row must come back finite; sampled blocks match
    the oracle."""
    B, H, nb, D = 1, 16, 512, 128
    S = nb * 64
    sv = S - 24
    g = torch.Generator(device="cpu").manual_seed(11)
    q, k, v = (torch.randn(B, H, S, D, generator=g).mul_(0.5).to(torch.bfloat16).to(DEV) for _ in range(3))
    rng = np.random.default_rng(12)
    keep = rng.random((B, H, nb, nb)) < rng.uniform(0.02, 0.3, size=(B, H, nb, 1))   # lengths vary by row
    keep[:, :, np.arange(nb), np.arange(nb)] = True
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    out = torch.full_like(q, float("nan"))
    rp, ci = gpu_lib.mask_to_csr(mask)
    gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=sv, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :, :sv]).all()
    blocks = [(0, h, i) for h in (0, 7, 15) for i in (0, 1, 200, nb - 1)]
    ref = oracle_attention_blocks(q, k, v, keep, blocks, sv)
    mx, mean = attention_errors(out, ref)
    print(f"[head order] max err {mx:.3e}, mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


# ----------------------------------------------------------------------------- near-threshold flags
def _check_near(flags, E, thr, name):
    """GPU flags against the oracle's band |E - (1 - thr)| <= 1e-6, except entries whose
    distance from the threshold lies within 1e-9 of the band edge (fixed-point vs fp64 E)."""
    f = flags.cpu().numpy().astype(bool)
    d = np.abs(E - (1.0 - thr))
    ref = d <= NEAR
    edge = np.abs(d - NEAR) <= 1e-9
    bad = (f != ref) & ~edge
    print(f"[near] {name}: flagged {int(f.sum())}, oracle {int(ref.sum())}, mismatches {int(bad.sum())}, "
          f"edge entries {int(edge.sum())}", flush=True)
    assert not bad.any()


@pytest.mark.parametrize("nb", [37, 300])
def test_near_threshold_flags_equal_rows(gpu_lib, nb):
    """q = 0: every row is uniform (p = 1/nb), so E = rank / nb exactly known. thr puts
    1 - thr at 4e-7 from the E of rank 11 (flagged) and 3e-6 from that of rank 20 (not
    flagged); nb = 37 runs the short-row select, nb = 300 the wide one."""
    B, H, D = 1, 2, 128
    q = torch.zeros(B, H, nb * 64, D, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(B, H, nb * 64, D, device=DEV).to(torch.bfloat16)
    for thr in (1 - (11 / nb + 4e-7), 1 - (20 / nb - 3e-6), 0.0, 0.5):
        m, nf = gpu_lib.nabla_build_mask(q, k, thr, near=True)
        m0 = gpu_lib.nabla_build_mask(q, k, thr)
        torch.cuda.synchronize()
        assert torch.equal(m, m0)
        keep, E = oracle_masks(q, k, thr)
        assert compare_masks(m, keep, E, thr)[0] == 0
        _check_near(nf, E, thr, f"uniform nb {nb} thr {thr:.9f}")
        if thr == 1 - (11 / nb + 4e-7):
            assert int(nf.sum()) == B * H * nb     # rank 11 of every row


@pytest.mark.parametrize("cid,heads", [(2, 4), (3, 4)])
def test_near_threshold_flags_random(gpu_lib, cid, heads):
    """Seeded workload inputs; thr = 0 flags the tail of each row (entries after the first
    1 - 1e-6 of the mass), thr 0.2 / the config's threshold flags few or none; the mask is
    the same with and without the flags; the sliding-tile and list entry points give the
    same flags (they describe the adaptive rule only)."""
    cfg = get_config(cid, heads)
    q, k, _ = make_inputs(cfg, seed=2, device=DEV)
    for thr in (0.0, 0.2) + tuple(cfg.thrs):
        m, nf = gpu_lib.nabla_build_mask(q, k, thr, near=True)
        torch.cuda.synchronize()
        keep, E = oracle_masks(q, k, thr)
        assert compare_masks(m, keep, E, thr)[0] == 0
        assert torch.equal(m, gpu_lib.nabla_build_mask(q, k, thr))
        _check_near(nf, E, thr, f"{cfg.name} thr {thr}")
        if cfg.sta is not None:
            ms, nfs = gpu_lib.nabla_build_mask_sta(q, k, thr, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                                   order_tile=cfg.order_tile, s_valid=cfg.S_valid, near=True)
            torch.cuda.synchronize()
            assert torch.equal(nfs, nf)
        if cfg.nb <= 256:
            nfl = torch.empty_like(nf)
            gpu_lib.nabla_build_mask_lists(q, k, thr, s_valid=cfg.S_valid, near=nfl)
            torch.cuda.synchronize()
            assert torch.equal(nfl, nf)
    _, nf8, _, _ = gpu_lib.nabla_build_mask_fp8(q, k, 0.0, near=True)
    torch.cuda.synchronize()
    assert torch.equal(nf8, gpu_lib.nabla_build_mask(q, k, 0.0, near=True)[1])


@pytest.mark.parametrize("nb", [257, 700, 1216, 1217])
def test_long_row_select_bounds(gpu_lib, nb):
    """Rows past the short-row limit (nb > 256) take the register-resident select: 3 column
    tiles per wave at nb 257, 6 at 700, 10 at 1216 and 1217 (a ragged last tile). Thresholds
    (0 keeps every block with mass), Top-k and an OR'd plane; D 128 and 64."""
    from dataclasses import replace
    for D in (128, 64):
        cfg = replace(get_config(3, heads=2), cid=9, name=f"long-{nb}", grid=(1, nb, 64), D=D)
        assert cfg.nb == nb and cfg.S_valid == cfg.S
        q, k, _ = make_inputs(cfg, seed=nb + D, device=DEV)
        rng = np.random.default_rng(nb)
        plane = rng.random((nb, nb)) < 0.03
        plane_t = torch.from_numpy(plane.astype(np.uint8)).to(DEV)
        for thr in (0.0, 0.1, 0.2, 0.6):
            m = gpu_lib.nabla_build_mask(q, k, thr)
            mo = gpu_lib.nabla_build_mask(q, k, thr, or_mask=plane_t)
            torch.cuda.synchronize()
            keep, E = oracle_masks(q, k, thr)
            bad, near = compare_masks(m, keep, E, thr)
            print(f"[long] nb {nb} D {D} thr {thr}: mismatches {bad}, near {near}, kept {keep.mean():.4f}", flush=True)
            assert bad == 0
            keep_or, _ = oracle_masks(q, k, thr, or_plane=plane)
            assert compare_masks(mo, keep_or, E, thr)[0] == 0
        for topk in (1, 37, nb - 1):
            mt = gpu_lib.nabla_build_mask_topk(q, k, topk)
            torch.cuda.synchronize()
            for h in range(cfg.H):
                ref, P = oracle.topk_mask(f64(q[0, h]), f64(k[0, h]), 64, topk)
                diff = mt[0, h].cpu().numpy().astype(bool) != ref
                kth = -np.sort(-P, axis=1)[:, topk - 1]
                assert not (diff & ~(np.abs(P - kth[:, None]) <= 2.0 ** -59)).any(), (topk, h)


def test_long_row_select_exact_ties(gpu_lib):
    """Long rows (nb = 300) whose key blocks repeat in threes: every reduced-map value occurs
    three times exactly, so the pivot's bucket holds tied keys that only the column index
    orders (descending p, then ascending index); in head 1 (q = 0) all 300 entries of a row
    tie. Thresholds and Top-k counts that fall inside a tie group."""
    from dataclasses import replace
    nb = 300
    cfg = replace(get_config(3, heads=2), cid=9, name="ties-300", grid=(1, nb, 64), D=128)
    q, k, _ = make_inputs(cfg, seed=77, device=DEV)
    kb = k.view(cfg.B, cfg.H, nb, 64, cfg.D)
    kb[:, :, 100:200] = kb[:, :, 0:100]
    kb[:, :, 200:300] = kb[:, :, 0:100]
    q[:, 1] = 0   # head 1: every entry of a row ties (more than a gathered bucket holds)
    for thr in (0.02, 0.05, 0.2, 0.5):
        m = gpu_lib.nabla_build_mask(q, k, thr)
        torch.cuda.synchronize()
        keep, E = oracle_masks(q, k, thr)
        bad, near = compare_masks(m, keep, E, thr)
        print(f"[ties] thr {thr}: mismatches {bad}, near {near}, kept {keep.mean():.4f}", flush=True)
        assert bad == 0
    for topk in (1, 2, 50, 100, 151):
        mt = gpu_lib.nabla_build_mask_topk(q, k, topk)
        torch.cuda.synchronize()
        for h in range(cfg.H):
            ref, P = oracle.topk_mask(f64(q[0, h]), f64(k[0, h]), 64, topk)
            diff = mt[0, h].cpu().numpy().astype(bool) != ref
            kth = -np.sort(-P, axis=1)[:, topk - 1]   # entries within 2^-59 of the k-th may swap
            assert not (diff & ~(np.abs(P - kth[:, None]) <= 2.0 ** -59)).any(), (topk, h)
            assert np.all(mt[0, h].sum(dim=-1).cpu().numpy() == topk)
