"""GPU parity of the fp8 e4m3fn block quantisation (standalone and fused into the mask
build) against the oracle's quantiser: codes and scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from parity_util import MAX_ERR, MEAN_ERR, attention_errors, f64, oracle_attention_blocks

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_codes(codes, scales, x):
    rc, rs = oracle.quantize_blocks(x.float().cpu().numpy(), 64)
    gs = scales.cpu().numpy()
    gc = codes.cpu().numpy()
    assert np.array_equal(gs, rs), f"scales differ at {np.argwhere(gs != rs)[:5]}"
    bad = np.argwhere(gc != rc)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:5]}: gpu {gc[tuple(bad[0])]} oracle {rc[tuple(bad[0])]}"


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128)])
def test_quantize_random_blocks(gpu_lib, dtype, D):
    g = torch.Generator(device="cpu").manual_seed(D)
    B, H, S = 2, 3, 640
    x = torch.randn(B, H, S, D, generator=g) * torch.exp(torch.randn(B, H, S // 64, 1, 1, generator=g) * 3).repeat_interleave(64, 2).reshape(B, H, S, 1)
    x[0, 1, 128:192] = 0                                  # an all-zero block
    x[1, 2, 5, 7] = 3e4                                   # one large outlier in a block
    x[1, 0, 70, :] = 1e-30                                # tiny values (code 0 after scaling)
    x = x.to(dtype).to(DEV)
    codes, scales = gpu_lib.quantize_fp8_blocks(x)
    torch.cuda.synchronize()
    _check_codes(codes, scales, x)


def test_quantize_strided_input(gpu_lib):
    g = torch.Generator(device="cpu").manual_seed(9)
    big = torch.randn(1, 4, 256, 256, generator=g).to(torch.bfloat16).to(DEV)
    x = big[:, 1:3, :, 64:192]                            # head and row strides of the parent
    codes, scales = gpu_lib.quantize_fp8_blocks(x)
    torch.cuda.synchronize()
    _check_codes(codes, scales, x)


def test_fused_mask_and_quantisation_config5(gpu_lib):
    cfg = get_config(5, heads=4)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    sta = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                 order_tile=cfg.order_tile, device=DEV)
    for thr in cfg.thrs[:2]:
        print(f"[fp8] config 5 ({cfg.H} heads) thr {thr}", flush=True)
        m_ref = gpu_lib.nabla_build_mask(q, k, thr, or_mask=sta)
        m, (q8, qs), (k8, ks) = gpu_lib.nabla_build_mask_fp8(q, k, thr, or_mask=sta)
        torch.cuda.synchronize()
        assert torch.equal(m, m_ref)
        _check_codes(q8, qs, q)
        _check_codes(k8, ks, k)
    # attention on the library's codes against the oracle on the dequantised values
    out = gpu_lib.block_sparse_attn_fwd(q8, k8, v, m, s_valid=cfg.S_valid, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    keep = m.cpu().numpy().astype(bool)
    vals = oracle.decode_e4m3fn(q8.cpu().numpy()), oracle.decode_e4m3fn(k8.cpu().numpy())
    q_deq = vals[0].reshape(1, cfg.H, cfg.nb, 64, cfg.D) * qs.cpu().numpy()[..., None, None]
    k_deq = vals[1].reshape(1, cfg.H, cfg.nb, 64, cfg.D) * ks.cpu().numpy()[..., None, None]
    blocks = [(0, h, i) for h in (0, cfg.H - 1) for i in (0, cfg.nb // 2, cfg.nb - 1)]
    ref = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid,
                                  q_deq=q_deq.reshape(1, cfg.H, cfg.S, cfg.D), k_deq=k_deq.reshape(1, cfg.H, cfg.S, cfg.D))
    mx, mean = attention_errors(out, ref)
    print(f"  fp8 attention on library codes: max {mx:.3e} mean {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


# --------------------------------------------------------------------------- incoherent processing
def _check_rotated(codes, scales, x, signs, key_side):
    rc, rs = oracle.quantize_blocks_rotated(x.float().cpu().numpy(), signs, key_side, 64)
    gs, gc = scales.cpu().numpy(), codes.cpu().numpy()
    assert np.array_equal(gs, rs), f"scales differ at {np.argwhere(gs != rs)[:5]}"
    bad = np.argwhere(gc != rc)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:5]}: gpu {gc[tuple(bad[0])]} oracle {rc[tuple(bad[0])]}"


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128),
                                     (torch.float32, 64)])
@pytest.mark.parametrize("key_side", [False, True])
def test_quantize_rotated_random_blocks(gpu_lib, dtype, D, key_side):
    from synth import make_signs
    g = torch.Generator(device="cpu").manual_seed(100 + D)
    B, H, S = 2, 3, 640
    x = torch.randn(B, H, S, D, generator=g) * torch.exp(torch.randn(B, H, S // 64, 1, 1, generator=g) * 3).repeat_interleave(64, 2).reshape(B, H, S, 1)
    x[0, 1, 128:192] = 0                                  # an all-zero block
    x[1, 2, 5, 7] = 3e4                                   # one large outlier in a block
    x[0, 0, :, 3] *= 40                                   # an outlier channel in every row of a head
    x = x.to(dtype).to(DEV)
    signs = make_signs(D, seed=D + key_side)
    codes, scales = gpu_lib.quantize_fp8_blocks_rotated(x, signs, key_side)
    torch.cuda.synchronize()
    _check_rotated(codes, scales, x, signs, key_side)


def test_fused_mask_and_rotated_quantisation_config5(gpu_lib):
    """The mask build's rotated fp8 codes (config 5 shape, 4 heads): the mask equals the
    unrotated build's, the codes and scales equal the oracle's bit for bit, and the attention
    on them matches the oracle on the dequantised rotated values."""
    from synth import make_signs
    cfg = get_config(5, heads=4)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    signs = make_signs(cfg.D, seed=0)
    thr = cfg.thrs[0]
    print(f"[fp8 rotated] config 5 ({cfg.H} heads) thr {thr}", flush=True)
    m_ref = gpu_lib.nabla_build_mask(q, k, thr)
    m, (q8, qs), (k8, ks) = gpu_lib.nabla_build_mask_fp8_rotated(q, k, thr, signs)
    torch.cuda.synchronize()
    assert torch.equal(m, m_ref)
    _check_rotated(q8, qs, q, signs, False)
    _check_rotated(k8, ks, k, signs, True)
    out = gpu_lib.block_sparse_attn_fwd(q8, k8, v, m, s_valid=cfg.S_valid, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    keep = m.cpu().numpy().astype(bool)
    shp = (1, cfg.H, cfg.nb, 64, cfg.D)
    q_deq = oracle.decode_e4m3fn(q8.cpu().numpy()).reshape(shp) * qs.cpu().numpy()[..., None, None]
    k_deq = oracle.decode_e4m3fn(k8.cpu().numpy()).reshape(shp) * ks.cpu().numpy()[..., None, None]
    blocks = [(0, h, i) for h in (0, cfg.H - 1) for i in (0, cfg.nb // 2, cfg.nb - 1)]
    ref = oracle_attention_blocks(q, k, v, keep, blocks, cfg.S_valid,
                                  q_deq=q_deq.reshape(1, cfg.H, cfg.S, cfg.D), k_deq=k_deq.reshape(1, cfg.H, cfg.S, cfg.D))
    mx, mean = attention_errors(out, ref)
    print(f"  rotated fp8 attention on library codes: max {mx:.3e} mean {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR


def test_rotation_lowers_fp8_attention_error_with_outlier_channels(gpu_lib):
    """What the rotation is for (FlashAttention-3 abstract: lower fp8 error): with a few
    outlier channels in Q and K, the GPU's fp8 attention on rotated codes lies closer to the
    fp64 oracle on the exact bf16 inputs than the GPU's fp8 attention on plain codes."""
    from synth import make_signs
    g = torch.Generator(device="cpu").manual_seed(7)
    B, H, S, D = 1, 2, 1024, 128
    q, k, v = (torch.randn(B, H, S, D, generator=g) for _ in range(3))
    for x in (q, k):
        x[..., [5, 40, 99]] *= 30.0                       # three outlier channels
    q, k = q * 0.12, k * 0.12                             # scores of order one
    q, k, v = (x.to(torch.bfloat16).to(DEV) for x in (q, k, v))
    nb = S // 64
    mask = torch.ones(B, H, nb, nb, dtype=torch.uint8, device=DEV)
    signs = make_signs(D, seed=3)
    pq, pk = gpu_lib.quantize_fp8_blocks(q), gpu_lib.quantize_fp8_blocks(k)
    rq = gpu_lib.quantize_fp8_blocks_rotated(q, signs, False)
    rk = gpu_lib.quantize_fp8_blocks_rotated(k, signs, True)
    o_plain = gpu_lib.block_sparse_attn_fwd(pq[0], pk[0], v, mask, q_scale=pq[1], k_scale=pk[1])
    o_rot = gpu_lib.block_sparse_attn_fwd(rq[0], rk[0], v, mask, q_scale=rq[1], k_scale=rk[1])
    torch.cuda.synchronize()
    keep = np.ones((nb, nb), dtype=bool)
    blocks = [(0, h, i) for h in range(H) for i in (0, 5, nb - 1)]
    ref = oracle_attention_blocks(q, k, v, keep[None, None].repeat(H, 1), blocks, S)
    e_plain = attention_errors(o_plain, ref)[1]
    e_rot = attention_errors(o_rot, ref)[1]
    print(f"  mean error against the exact inputs: plain fp8 {e_plain:.3e}, rotated fp8 {e_rot:.3e}", flush=True)
    assert e_rot < 0.75 * e_plain, (e_plain, e_rot)


def test_quantize_rotated_strided_input(gpu_lib):
    from synth import make_signs
    g = torch.Generator(device="cpu").manual_seed(19)
    big = torch.randn(1, 4, 256, 256, generator=g).to(torch.bfloat16).to(DEV)
    x = big[:, 1:3, :, 64:192]                            # head and row strides of the parent
    signs = make_signs(128, seed=5)
    for key_side in (False, True):
        codes, scales = gpu_lib.quantize_fp8_blocks_rotated(x, signs, key_side)
        torch.cuda.synchronize()
        _check_rotated(codes, scales, x, signs, key_side)


def test_fused_rotated_f32_d64(gpu_lib):
    """The fused rotated quantisation with f32 inputs at D = 64 (the tiny config's shape):
    mask equal to the unrotated build's, codes and scales bit-exact."""
    from synth import make_signs
    cfg = get_config(1)
    q, k, v = make_inputs(cfg, seed=3, device=DEV)
    signs = make_signs(cfg.D, seed=1)
    m_ref = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0])
    m, (q8, qs), (k8, ks) = gpu_lib.nabla_build_mask_fp8_rotated(q, k, cfg.thrs[0], signs)
    torch.cuda.synchronize()
    assert torch.equal(m, m_ref)
    _check_rotated(q8, qs, q, signs, False)
    _check_rotated(k8, ks, k, signs, True)
