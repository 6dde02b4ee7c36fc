"""The checked build (libbsa_checked.so, compiled with -DBSA_CHECKED) on valid inputs.

Its kernels test every index they read from list data (kv-list entries, list lengths,
bit-row entries, backward list entries) and record a failed test in a device flag word
instead of touching memory out of bounds. On the benchmark step's calls -- the short-row
list path (2B-DiT shape), the long-row path with pairing offsets, bit rows and the work
order each workgroup derives (14B shape, 2 heads), the kv lists handed in by the caller,
fp8 Q/K, the kv-chunked walk and the backward -- no flag may be set, and every output must equal the production
library's bit for bit (the tests compile away there)."""
import contextlib

import pytest
import torch

import block_sparse_attention_mask_amd as bsa
from synth import get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@contextlib.contextmanager
def _library(path):
    """Run the binding against the library at `path`, then restore the production one."""
    saved = bsa._lib, bsa._lib_path
    try:
        yield bsa.load(path)
    finally:
        bsa._lib, bsa._lib_path = saved


def _step(cfg, q, k, v):
    """The calls of a benchmark step plus the backward; returns every output."""
    thr = cfg.thrs[0]
    outs = {}
    if cfg.nb <= 256:
        sta_kw = dict(grid=cfg.grid, tile=cfg.sta.tile, window=cfg.sta.window, order=cfg.order,
                      order_tile=cfg.order_tile)
        m, kv_len, kv_idx, wo = bsa.nabla_build_mask_lists(q, k, thr, s_valid=cfg.S_valid, **sta_kw)
        outs["lists"] = bsa.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid)
    else:
        m = bsa.nabla_build_mask(q, k, thr)
    rp, ci = bsa.mask_to_csr(m)
    outs["mask"] = m
    outs["csr"] = bsa.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=cfg.S_valid)
    o, lse = bsa.block_sparse_attn_fwd(q, k, v, m, s_valid=cfg.S_valid, return_lse=True)
    outs["o"], outs["lse"] = o, lse
    # fp8 Q/K (codes and scales from the mask build's own read) through the same attention
    m8, (q8, qs), (k8, ks) = bsa.nabla_build_mask_fp8(q, k, thr)
    outs["fp8"] = bsa.block_sparse_attn_fwd(q8, k8, v, m8, s_valid=cfg.S_valid, q_scale=qs, k_scale=ks)
    # the kv-chunked walk and its combine
    bsa.set_attn_kv_chunk(7)
    try:
        outs["chunked"] = bsa.block_sparse_attn_fwd_csr(q, k, v, rp, ci, s_valid=cfg.S_valid)
    finally:
        bsa.set_attn_kv_chunk(0)
    g = torch.Generator(device=DEV).manual_seed(5)
    do = (torch.randn(q.shape, generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    outs["dq"], outs["dk"], outs["dv"] = bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, m, s_valid=cfg.S_valid)
    torch.cuda.synchronize()
    return {key: val.clone() for key, val in outs.items()}


@pytest.mark.parametrize("cid,heads", [(2, 16), (3, 2)])
def test_checked_build_sets_no_flag_and_matches(gpu_lib, cid, heads):
    cfg = get_config(cid, heads=heads)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    print(f"[checked] {cfg.name} ({heads} heads, nb {cfg.nb})", flush=True)
    ref = _step(cfg, q, k, v)
    assert gpu_lib.load().bsa_checked_build() == 0
    assert gpu_lib.load().bsa_check_flags(1) == 0
    with _library(bsa.CHECKED_LIB_PATH) as chk:
        assert chk.bsa_checked_build() == 1
        assert chk.bsa_check_flags(1) == 0
        got = _step(cfg, q, k, v)
        flags = chk.bsa_check_flags(1)
    assert flags == 0, f"checked build flagged {flags:#x}"
    for key in ref:
        assert torch.equal(ref[key], got[key]), key
