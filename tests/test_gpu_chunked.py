"""GPU parity of the kv-chunked attention walk (bsa_set_attn_kv_chunk): every (head, chunk,
query-block pair) is a work item leaving a partial state, merged by a combine launch.

Online softmax is associative, so the chunked walk must match the oracle to the same
tolerances as the whole-row walk (max |err| <= 2e-2, mean <= 2e-3 for bf16 inputs), with
lse within the bf16 normaliser bound, for chunk widths that cut rows into ragged parts,
on empty rows, padded tails, D = 64 and 128, and bf16, f32 and fp8 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs, quantize_fp8_blocks
from parity_util import MAX_ERR, MEAN_ERR, attention_errors, f64, oracle_attention_blocks, oracle_masks

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def chunked(gpu_lib):
    """Yields a setter of the chunk width; restores whole rows afterwards."""
    yield gpu_lib.set_attn_kv_chunk
    gpu_lib.set_attn_kv_chunk(0)


@pytest.mark.parametrize("w", [1, 3, 64])
def test_chunked_config2_full(gpu_lib, chunked, w):
    """The 2B-DiT workload (16 heads, 128 blocks, NABLA | sliding tiles), every query block
    against the oracle; the chunked result is deterministic and the CSR and mask entries
    agree bit for bit."""
    cfg = get_config(2)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    sta = oracle.sta_block_mask(cfg.grid, cfg.order, cfg.order_tile, cfg.sta.tile, cfg.sta.window, 64, cfg.S)
    keep, _ = oracle_masks(q, k, 0.1, or_plane=sta)
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    assert chunked(w) == 0
    out, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, return_lse=True)
    out, lse = out.clone(), lse.clone()
    again = gpu_lib.block_sparse_attn_fwd(q, k, v, mask).clone()
    rp, ci = gpu_lib.mask_to_csr(mask)
    via_csr = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci)
    torch.cuda.synchronize()
    assert torch.equal(out, again) and torch.equal(out, via_csr)
    blocks = [(0, h, i) for h in range(cfg.H) for i in range(cfg.nb)]
    ref = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid)
    mx, mean = attention_errors(out, ref)
    print(f"[chunked w={w}] {cfg.name}: max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR
    # against the whole-row walk: both within the tolerance of the oracle, and lse within
    # 5e-3 of each other (each within -log(1 - 2^-8) ~ 3.9e-3 of exact in the worst case;
    # the roundings of the two walks' normalisers are not all one way)
    chunked(0)
    whole, lse_w = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, return_lse=True)
    torch.cuda.synchronize()
    fin = torch.isfinite(lse_w)
    assert torch.equal(fin, torch.isfinite(lse))
    assert (lse[fin] - lse_w[fin]).abs().max().item() < 5e-3
    assert (out.float() - whole.float()).abs().mean().item() <= MEAN_ERR


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("w", [1, 2, 5])
def test_chunked_edge_rows(gpu_lib, chunked, D, w):
    """Empty rows, a row whose only block is the partly padded last one, a padded tail,
    an odd block count (a pair with one block), lists that skip whole chunks."""
    B, H, nb = 1, 2, 13
    S, Sv = 64 * nb, 64 * (nb - 1) + 7
    g = torch.Generator(device="cpu").manual_seed(100 * D + w)
    q, k, v = (torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    keep = np.random.default_rng(D + w).random((B, H, nb, nb)) < 0.3
    keep[0, 0, 2] = False                  # no kept block
    keep[0, 1, 3] = False
    keep[0, 1, 3, nb - 1] = True           # only the partly padded last block
    keep[0, 0, 5] = False
    keep[0, 0, 5, [0, nb - 2]] = True      # two blocks far apart: the chunks between are empty
    keep[0, 1, nb - 1] = False             # the odd last block, alone in its pair, empty
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    chunked(w)
    out, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, mask, s_valid=Sv, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out[0, 0, 128:192] == 0) and torch.isinf(lse[0, 0, 128:192]).all()
    assert torch.all(out[:, :, Sv:] == 0) and torch.isinf(lse[:, :, Sv:]).all()
    for h in range(H):
        O, L = oracle.block_sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), keep[0, h], 64, Sv)
        err = np.abs(f64(out[0, h]) - O)
        assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR
        fin = np.isfinite(L)
        assert np.array_equal(fin, np.isfinite(f64(lse[0, h])))
        # the normaliser is the sum of the bf16-rounded weights: |lse - exact| <= -log(1 - 2^-8)
        # (3.9e-3) in the worst case; held to 2.5e-3 here, inside that bound
        assert np.abs(f64(lse[0, h])[fin] - L[fin]).max() < 2.5e-3


def test_chunked_f32_and_fp8(gpu_lib, chunked):
    """f32 inputs (hi/lo split, f32 output) and fp8 e4m3 Q/K with per-block scales."""
    cfg = get_config(2, heads=3)
    q, k, v = make_inputs(cfg, seed=3, device=DEV)
    keep, _ = oracle_masks(q, k, 0.2)
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    blocks = [(0, h, i) for h in range(cfg.H) for i in range(0, cfg.nb, 5)]
    chunked(7)
    o32 = gpu_lib.block_sparse_attn_fwd(q.float(), k.float(), v.float(), mask)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    mx, mean = attention_errors(o32, oracle_attention_blocks(q.float(), k.float(), v.float(), keep, blocks,
                                                             cfg.S_valid))
    print(f"[chunked f32] max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR
    qc, qs = quantize_fp8_blocks(q)
    kc, ks = quantize_fp8_blocks(k)
    o8 = gpu_lib.block_sparse_attn_fwd(qc, kc, v, mask, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    nb, D = cfg.nb, cfg.D
    deq = lambda c, s, h: (c[0, h].view(torch.float8_e4m3fn).double().view(nb, 64, D)
                           * s[0, h].double()[:, None, None]).view(cfg.S, D).cpu().numpy()
    ref = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid, q_deq=lambda b, h: deq(qc, qs, h),
                                  k_deq=lambda b, h: deq(kc, ks, h))
    mx, mean = attention_errors(o8, ref)
    print(f"[chunked fp8] max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


def test_chunked_lists_entry_and_workspace(gpu_lib, chunked):
    """The fixed-stride lists entry gives the CSR entry's result bit for bit under the chunked
    walk, and the workspace query follows the setting."""
    import ctypes
    cfg = get_config(2, heads=4)
    q, k, v = make_inputs(cfg, seed=4, device=DEV)
    lib = gpu_lib.load()
    shp = gpu_lib._shape(q, cfg.S_valid)
    assert lib.attn_csr_workspace_size(ctypes.byref(shp), gpu_lib.BSA_BF16) == 0
    chunked(16)
    nch = (cfg.nb + 15) // 16
    rows = cfg.B * cfg.H * cfg.nb
    need = lib.attn_csr_workspace_size(ctypes.byref(shp), gpu_lib.BSA_BF16)
    assert need >= rows * nch * 64 * (4 * cfg.D + 8)
    mask, kv_len, kv_idx, _ = gpu_lib.nabla_build_mask_lists(q, k, 0.1, s_valid=cfg.S_valid)
    a = gpu_lib.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid).clone()
    rp, ci = gpu_lib.mask_to_csr(mask)
    b = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=cfg.S_valid)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_chunked_with_pairing_offsets(gpu_lib, chunked):
    """Rows long enough for pairing offsets (nb = 600, lists alike one offset apart): the
    chunked walk over offset pairs writes every block, matches the oracle on sampled blocks
    and the whole-row walk within the tolerances."""
    B, H, nb, D = 1, 2, 600, 128
    S = nb * 64
    sv = S - 30
    rng = np.random.default_rng(600)
    keep = np.zeros((B, H, nb, nb), bool)
    for h, d in enumerate((55, 1)):
        base = rng.random((d, nb)) < 0.08
        keep[0, h] = base[np.arange(nb) % d]
        keep[0, h, np.arange(nb), np.arange(nb)] = True
    mask = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    g = torch.Generator(device="cpu").manual_seed(600)
    q, k, v = (torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    rp, ci = gpu_lib.mask_to_csr(mask)
    assert gpu_lib.attn_pair_offsets(q, rp, ci, s_valid=sv).tolist() == [55, 1]
    chunked(64)
    out = torch.full_like(v, float("nan"))
    out = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=sv, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    blocks = [(0, h, i) for h in range(H) for i in (0, 1, 54, 55, 56, 299, 598, 599)]
    mx, mean = attention_errors(out, oracle_attention_blocks(q, k, v, keep, blocks, sv))
    print(f"[chunked + pairing] max err {mx:.3e} mean err {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR
    chunked(0)
    whole = gpu_lib.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=sv)
    torch.cuda.synchronize()
    assert (out.float() - whole.float()).abs().mean().item() <= MEAN_ERR
