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
