"""The whole step (sliding-tile mask, NABLA mask, kv lists, work order, attention) captured
as one HIP graph and replayed: every replay, with the program's own eager work and
synchronisations between replays, equals the eager step bit for bit."""
import ctypes

import pytest
import torch

from synth import get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _make_step(bsa, cfg, q, k, v, fp8, lists=False):
    nb, B, H = cfg.nb, cfg.B, cfg.H
    plane = torch.empty(nb, nb, dtype=torch.uint8, device=DEV)
    mask = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=DEV)
    rows = B * H * nb
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=DEV)
    col_idx = torch.empty(rows * nb, dtype=torch.int32, device=DEV)
    lib = bsa.load()
    shp = bsa.Shape(B, H, cfg.S, cfg.S_valid, cfg.D, 64)
    csr_ws = torch.empty(max(256, lib.csr_workspace_size(B, H, nb)), dtype=torch.uint8, device=DEV)
    code = bsa.BSA_FP8_E4M3FN if fp8 else bsa.BSA_BF16
    attn_ws = torch.empty(max(256, lib.attn_csr_workspace_size(ctypes.byref(shp), code)), dtype=torch.uint8,
                          device=DEV)
    n_slots = lib.attn_work_order_slots(ctypes.byref(shp))
    wo = torch.empty(max(n_slots, 1), dtype=torch.int32, device=DEV)
    out = torch.empty_like(v)
    q8, k8 = torch.empty(q.shape, dtype=torch.uint8, device=DEV), torch.empty(k.shape, dtype=torch.uint8, device=DEV)
    qs = torch.empty(B, H, nb, dtype=torch.float32, device=DEV)
    ks = torch.empty(B, H, nb, dtype=torch.float32, device=DEV)
    kv_len = torch.empty(rows, dtype=torch.int32, device=DEV)
    kv_idx = torch.empty(rows, nb, dtype=torch.int32, device=DEV)
    lists_ws = bsa.nabla_lists_workspace(q, cfg.S_valid)

    def step_lists():
        # mask, kv lists from the mask build; attention derives its work order from kv_len
        bsa.nabla_build_mask_lists(q, k, cfg.thrs[0], cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                   order_tile=cfg.order_tile, s_valid=cfg.S_valid,
                                   out=(mask, kv_len, kv_idx, None), ws=lists_ws)
        bsa.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid, out=out, ws=attn_ws)

    def step():
        bsa.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                           order_tile=cfg.order_tile, device=DEV, out=plane)
        if fp8:
            bsa.nabla_build_mask_fp8(q, k, cfg.thrs[0], or_mask=plane, out=mask, q8_out=(q8, qs), k8_out=(k8, ks))
        else:
            bsa.nabla_build_mask(q, k, cfg.thrs[0], or_mask=plane, out=mask)
        rp, ci = bsa.mask_to_csr(mask, row_ptr=row_ptr, col_idx=col_idx, ws=csr_ws)
        w = bsa.attn_work_order(q, rp, s_valid=cfg.S_valid, out=wo) if n_slots > 0 else None
        bsa.block_sparse_attn_fwd_csr(q8 if fp8 else q, k8 if fp8 else k, v, rp, ci, s_valid=cfg.S_valid,
                                      q_scale=qs if fp8 else None, k_scale=ks if fp8 else None, out=out,
                                      ws=attn_ws, work_order=w)
    return (step_lists if lists else step), out, mask


@pytest.mark.parametrize("mode", ["bf16", "fp8", "lists"])
def test_step_graph_replays_match_eager(gpu_lib, mode):
    fp8 = mode == "fp8"
    cfg = get_config(2, heads=4)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    step, out, mask = _make_step(gpu_lib, cfg, q, k, v, fp8, lists=mode == "lists")
    step()
    torch.cuda.synchronize()
    ref, ref_mask = out.clone(), mask.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.zero_()
        mask.fill_(7)
        eager = gpu_lib.block_sparse_attn_fwd(q, k, v, ref_mask, s_valid=cfg.S_valid)   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] {mode} replay {r}", flush=True)
        assert torch.equal(mask, ref_mask)
        assert torch.equal(out, ref)
        del eager
    # the graph reads its inputs at replay time: change them in place, compare with an eager step
    q.mul_(0.5)
    g.replay()
    torch.cuda.synchronize()
    got = out.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(got, out)
    assert not torch.equal(got, ref)
