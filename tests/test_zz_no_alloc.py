"""The allocation-free mask entry point (nabla_build_mask_noalloc) against nabla_build_mask.

nabla_build_mask_noalloc runs the same kernels with the library's static per-GPU scratch
array as workspace. Two calls in a row on one GPU, the second with a smaller input (the
array still holds the first call's pooled vectors), each compared bit for bit with the
workspace-taking entry point on the same inputs: the long-row select (nb = 1182) and the
short-row one (nb = 128), with near-threshold flags and an OR'd sliding-tile mask.
"""
import pytest
import torch

from synth import get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_noalloc_two_calls_match_the_workspace_entry_point(gpu_lib):
    cases = [(get_config(3, heads=12), 0.2), (get_config(2, heads=3), 0.1)]
    for cfg, thr in cases:
        q, k, _ = make_inputs(cfg, seed=7, device=DEV)
        plane = None
        if cfg.sta is not None:
            plane = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window,
                                           order=cfg.order, order_tile=cfg.order_tile, device=DEV)
        ref, near_ref = gpu_lib.nabla_build_mask(q, k, thr, or_mask=plane, near=True)
        out = torch.full_like(ref, 7)
        nf = torch.full_like(ref, 7)
        gpu_lib.nabla_build_mask_noalloc(q, k, thr, or_mask=plane, out=out, near=nf)
        plain = gpu_lib.nabla_build_mask_noalloc(q, k, thr, or_mask=plane)
        torch.cuda.synchronize()
        print(f"[noalloc] {cfg.name} nb {cfg.nb} thr {thr}: kept {ref.float().mean().item():.4f}, "
              f"flagged {int(near_ref.sum().item())}", flush=True)
        assert torch.equal(out, ref)
        assert torch.equal(nf, near_ref)
        assert torch.equal(plain, ref)


def test_noalloc_rejects_more_than_its_scratch(gpu_lib):
    cfg = get_config(2, heads=1)
    q, k, _ = make_inputs(cfg, seed=0, device=DEV)
    big = q.expand(1, 600, cfg.S, cfg.D)          # 600 heads of 8192 tokens: 157 MB of scratch
    with pytest.raises(gpu_lib.BsaError, match="scratch"):
        gpu_lib.nabla_build_mask_noalloc(big, big, 0.1)
