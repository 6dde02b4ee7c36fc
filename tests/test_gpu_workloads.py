"""GPU parity at the full benchmark workloads, through the calls the benchmark step makes.

Each case builds every head's mask on the GPU and compares it with the oracle's bit for
bit (blocks within 1e-6 of the threshold excused and counted). The attention then runs
on the ORACLE's mask, through the same entry points and in the same launch form as the
benchmark step (kv lists from bsa_mask_to_csr, block_sparse_attn_fwd_csr with the
order each workgroup derives in the kernel), into an output that starts as NaN: every
valid row must be written, and the sampled query blocks -- all blocks of heads 0 and
H-1 and at least 16 seeded blocks of every other head, always with its first, last,
densest and sparsest rows -- must match the oracle within max |err| <= 2e-2 and
mean |err| <= 2e-3 (bf16 inputs; the fp8 run against the oracle fed the dequantised
codes the library itself produced).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from parity_util import (MAX_ERR, MEAN_ERR, attention_errors, compare_masks, f64, masks_from_probs,
                         oracle_attention_blocks, oracle_probs, sample_blocks)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sta_plane(cfg):
    return oracle.sta_block_mask(cfg.grid, cfg.order, cfg.order_tile, cfg.sta.tile, cfg.sta.window, 64, cfg.S)


def _attention_as_benchmarked(bsa, cfg, qa, ka, v, keep, q_scale=None, k_scale=None):
    """The benchmark's attention call on the given mask; returns the output (NaN-initialised)."""
    mask = torch.from_numpy(np.ascontiguousarray(keep, dtype=np.uint8)).to(DEV)
    rp, ci = bsa.mask_to_csr(mask)
    out = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bsa.block_sparse_attn_fwd_csr(qa, ka, v, rp, ci, s_valid=cfg.S_valid, q_scale=q_scale, k_scale=k_scale, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :, :cfg.S_valid]).all(), "some valid query rows were not written"
    assert torch.all(out[:, :, cfg.S_valid:] == 0)
    return out


def _check_blocks(name, out, ref):
    mx, mean = attention_errors(out, ref)
    print(f"[{name}] {len(ref)} query blocks: max err {mx:.3e}, mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR, (mx, mean)


def _derives_head_order(bsa, q, cfg):
    # the shapes here make many rounds of long rows: no work-order array, each workgroup
    # derives its item (longest first inside its head) in the kernel, as in the bench step
    return bsa.attn_work_order_slots(q, s_valid=cfg.S_valid) == 0 and cfg.nb >= 512


@pytest.mark.timeout(1200)
def test_config3_all_heads_as_benchmarked(gpu_lib):
    """14B 720p shape: 40 heads, NABLA thr 0.2, every head with its real mask."""
    cfg = get_config(3)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    thr = cfg.thrs[0]
    print(f"[cfg3] {cfg.name}: B {cfg.B} H {cfg.H} nb {cfg.nb} thr {thr}", flush=True)
    m = gpu_lib.nabla_build_mask(q, k, thr)
    torch.cuda.synchronize()
    P = oracle_probs(q, k)
    keep, E = masks_from_probs(P, thr)
    bad, near = compare_masks(m, keep, E, thr, P=P)
    print(f"[cfg3] mask: mismatches {bad}, near-threshold {near}, kept {keep.mean():.4f}", flush=True)
    assert bad == 0
    assert _derives_head_order(gpu_lib, q, cfg)
    out = _attention_as_benchmarked(gpu_lib, cfg, q, k, v, keep)
    blocks = sample_blocks(keep, 16, seed=31, full_heads=(0, cfg.H - 1))
    _check_blocks("cfg3", out, oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid))


@pytest.mark.timeout(900)
def test_config4_all_heads(gpu_lib):
    """HunyuanVideo-like shape: 24 heads, the static sliding-tile mask (built by the library)."""
    cfg = get_config(4)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    plane = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                   order_tile=cfg.order_tile, device=DEV)
    ref_plane = _sta_plane(cfg)
    assert np.array_equal(plane.cpu().numpy().astype(bool), ref_plane)
    keep = np.broadcast_to(ref_plane, (cfg.B, cfg.H, cfg.nb, cfg.nb))
    assert _derives_head_order(gpu_lib, q, cfg)
    out = _attention_as_benchmarked(gpu_lib, cfg, q, k, v, keep)
    blocks = sample_blocks(keep, 16, seed=41, full_heads=(0, cfg.H - 1))
    _check_blocks("cfg4", out, oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid))


@pytest.fixture(scope="module")
def sweep_data(gpu_lib):
    """Config 5 inputs and the oracle's reduced-map probabilities (shared by all its cases)."""
    cfg = get_config(5)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    P = oracle_probs(q, k)
    return cfg, q, k, v, P, _sta_plane(cfg)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("thr", [0.05, 0.1, 0.2, 0.4])
@pytest.mark.parametrize("qk", ["bf16", "fp8"])
def test_config5_sweep_all_heads(gpu_lib, sweep_data, thr, qk):
    """Combined sweep: NABLA at thr OR'd with sliding tiles (4x8x8 tiles, 3x3x3 window) on the
    row-major 21x45x80 grid, 40 heads; bf16 Q/K, and fp8 e4m3 Q/K with per-block scales
    produced by nabla_build_mask_fp8 from the same read that builds the mask."""
    cfg, q, k, v, P, plane = sweep_data
    assert thr in cfg.thrs
    sta = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                 device=DEV)
    keep, E = masks_from_probs(P, thr, or_plane=plane)
    if qk == "bf16":
        m = gpu_lib.nabla_build_mask(q, k, thr, or_mask=sta)
        qa, ka, qs, ks, qd, kd = q, k, None, None, None, None
    else:
        m, (qa, qs), (ka, ks) = gpu_lib.nabla_build_mask_fp8(q, k, thr, or_mask=sta)

        def deq(codes, scales):
            def per_head(b, h):
                c = codes[b, h].view(torch.float8_e4m3fn).to(torch.float64).view(cfg.nb, 64, cfg.D)
                return (c * scales[b, h].to(torch.float64)[:, None, None]).view(cfg.S, cfg.D).cpu().numpy()
            return per_head
        qd, kd = deq(qa, qs), deq(ka, ks)
    torch.cuda.synchronize()
    bad, near = compare_masks(m, keep, E, thr, P=P)
    print(f"[cfg5 {qk} thr {thr}] mask: mismatches {bad}, near-threshold {near}, kept {keep.mean():.4f}",
          flush=True)
    assert bad == 0
    assert _derives_head_order(gpu_lib, q, cfg)
    out = _attention_as_benchmarked(gpu_lib, cfg, qa, ka, v, keep, q_scale=qs, k_scale=ks)
    full = (0, cfg.H - 1) if (qk, thr) == ("bf16", 0.2) else ()
    blocks = sample_blocks(keep, 16, seed=int(thr * 100) + (7 if qk == "fp8" else 0), full_heads=full)
    _check_blocks(f"cfg5 {qk} thr {thr}", out,
                  oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid, q_deq=qd, k_deq=kd))


@pytest.mark.timeout(900)
def test_config5_fp8_rotated_all_heads(gpu_lib, sweep_data):
    """The fp8 sweep case with incoherent processing (thr 0.05, the fp8 bench threshold): the
    mask from nabla_build_mask_fp8_rotated equals the oracle's, the rotated codes and scales of
    heads 0 and H-1 equal the oracle's bit for bit, and the attention on the library's rotated
    codes matches the oracle fed their dequantised values on sampled blocks of every head."""
    from synth import make_signs
    cfg, q, k, v, P, plane = sweep_data
    thr = 0.05
    signs = make_signs(cfg.D, seed=0)
    sta = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                 device=DEV)
    keep, E = masks_from_probs(P, thr, or_plane=plane)
    m, (qa, qs), (ka, ks) = gpu_lib.nabla_build_mask_fp8_rotated(q, k, thr, signs, or_mask=sta)
    torch.cuda.synchronize()
    bad, near = compare_masks(m, keep, E, thr, P=P)
    print(f"[cfg5 fp8 rotated thr {thr}] mask: mismatches {bad}, near-threshold {near}", flush=True)
    assert bad == 0
    for h in (0, cfg.H - 1):
        for x, codes, scales, key in ((q, qa, qs, False), (k, ka, ks, True)):
            rc, rs = oracle.quantize_blocks_rotated(x[0, h].float().cpu().numpy(), signs, key, 64)
            assert np.array_equal(scales[0, h].cpu().numpy(), rs)
            assert np.array_equal(codes[0, h].cpu().numpy(), rc)

    def deq(codes, scales):
        def per_head(b, h):
            c = codes[b, h].view(torch.float8_e4m3fn).to(torch.float64).view(cfg.nb, 64, cfg.D)
            return (c * scales[b, h].to(torch.float64)[:, None, None]).view(cfg.S, cfg.D).cpu().numpy()
        return per_head
    out = _attention_as_benchmarked(gpu_lib, cfg, qa, ka, v, keep, q_scale=qs, k_scale=ks)
    blocks = sample_blocks(keep, 16, seed=12)
    _check_blocks(f"cfg5 fp8 rotated thr {thr}", out,
                  oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid, q_deq=deq(qa, qs), k_deq=deq(ka, ks)))
