"""GPU parity of the backward pass (through the C-ABI) against the fp64 gradient oracle.

The GPU forward supplies o and lse (the backward's contract); the oracle recomputes
everything in fp64 from the same bf16 inputs and the same mask. Per head and per
gradient: max |err| <= 4e-2 max |ref| and mean |err| <= 2e-3 max |ref|, over every row
where the oracle is cheap, else over sampled query blocks (dq) and key blocks (dk, dv)
that always include the first, middle and last (padded) ones.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from parity_util import GRAD_MAX_REL, GRAD_MEAN_REL, f64, grad_errors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(bsa, q, k, v, do, mask, s_valid, grad_dtype=None, scale=None):
    o, lse = bsa.block_sparse_attn_fwd(q, k, v, mask, s_valid=s_valid, scale=scale, return_lse=True)
    dq, dk, dv = bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, mask, s_valid=s_valid, scale=scale,
                                           grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check_head(name, gpu, ref, rows):
    mx, mean, scale = grad_errors(gpu, ref, rows)
    print(f"  {name}: max {mx:.3e} mean {mean:.3e} (max |ref| {scale:.3e})", flush=True)
    assert mx <= GRAD_MAX_REL * scale + 1e-6, name
    assert mean <= GRAD_MEAN_REL * scale + 1e-7, name


def _rows(blocks, S):
    return np.concatenate([np.arange(i * 64, min((i + 1) * 64, S)) for i in blocks])


def _random_case(B, H, S, D, s_valid, seed, density=0.4):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k, v, do = (torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(4))
    nb = S // 64
    m = (torch.rand(B, H, nb, nb, generator=g) < density)
    m[..., torch.arange(nb), torch.arange(nb)] = True
    m[0, 0, nb // 2] = False                              # a query block with no kept key block
    m[0, -1, 0] = True                                    # a fully kept row
    m[0, -1, :, min(1, nb - 1)] = True                    # a fully kept column
    return q, k, v, do, m.to(torch.uint8).to(DEV)


@pytest.mark.parametrize("S,D,s_valid,gdt", [
    (256, 64, 256, None), (256, 128, 230, None), (960, 128, 911, torch.float32), (1024, 64, 1000, torch.float32),
])
def test_backward_small_full(gpu_lib, S, D, s_valid, gdt):
    B, H = 2, 2
    q, k, v, do, m = _random_case(B, H, S, D, s_valid, seed=S + D)
    print(f"[bwd] S {S} D {D} S_valid {s_valid} grads {gdt or torch.bfloat16}", flush=True)
    dq, dk, dv = _run(gpu_lib, q, k, v, do, m, s_valid, grad_dtype=gdt)
    mk = m.cpu().numpy().astype(bool)
    rows = np.arange(S)
    for b in range(B):
        for h in range(H):
            rq, rk, rv = oracle.block_sparse_attention_bwd(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h]),
                                                           mk[b, h], 64, s_valid)
            _check_head(f"dq[{b},{h}]", dq[b, h], rq, rows)
            _check_head(f"dk[{b},{h}]", dk[b, h], rk, rows)
            _check_head(f"dv[{b},{h}]", dv[b, h], rv, rows)
            # rows that carry no gradient are exactly zero
            assert torch.all(dq[b, h, s_valid:] == 0) and torch.all(dk[b, h, s_valid:] == 0)
            assert torch.all(dv[b, h, s_valid:] == 0)


def test_backward_dense_mask_and_scale(gpu_lib):
    B, H, S, D = 1, 2, 512, 128
    q, k, v, do, _ = _random_case(B, H, S, D, S, seed=7)
    m = torch.ones(S // 64, S // 64, dtype=torch.uint8, device=DEV)      # one broadcast plane
    dq, dk, dv = _run(gpu_lib, q, k, v, do, m, S, scale=0.05)
    rows = np.arange(S)
    for h in range(H):
        rq, rk, rv = oracle.block_sparse_attention_bwd(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h]),
                                                       np.ones((S // 64, S // 64), bool), 64, S, scale=0.05)
        _check_head(f"dq[{h}]", dq[0, h], rq, rows)
        _check_head(f"dk[{h}]", dk[0, h], rk, rows)
        _check_head(f"dv[{h}]", dv[0, h], rv, rows)


def test_backward_config2_full(gpu_lib):
    cfg = get_config(2, heads=2)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    do = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(3)).to(torch.bfloat16).to(DEV)
    sta = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                 order_tile=cfg.order_tile, device=DEV)
    m = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0], or_mask=sta)
    print(f"[bwd] config 2, {cfg.H} heads, kept {m.float().mean().item():.4f}", flush=True)
    dq, dk, dv = _run(gpu_lib, q, k, v, do, m, cfg.S_valid)
    mk = m.cpu().numpy().astype(bool)
    rows = np.arange(cfg.S)
    for h in range(cfg.H):
        rq, rk, rv = oracle.block_sparse_attention_bwd(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h]),
                                                       mk[0, h], 64, cfg.S_valid)
        _check_head(f"dq[{h}]", dq[0, h], rq, rows)
        _check_head(f"dk[{h}]", dk[0, h], rk, rows)
        _check_head(f"dv[{h}]", dv[0, h], rv, rows)


@pytest.mark.parametrize("cid", [3, 4])
def test_backward_full_size_sampled(gpu_lib, cid):
    cfg = get_config(cid)
    q, k, v = make_inputs(cfg, seed=0, device=DEV)
    do = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(5)).to(torch.bfloat16).to(DEV)
    if cfg.thrs:
        m = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0])
    else:
        m = gpu_lib.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                   order_tile=cfg.order_tile, device=DEV)
    print(f"[bwd] config {cid} full size {tuple(q.shape)}", flush=True)
    dq, dk, dv = _run(gpu_lib, q, k, v, do, m, cfg.S_valid)
    mk = m.cpu().numpy().astype(bool)
    if mk.ndim == 2:
        mk = np.broadcast_to(mk, (cfg.B, cfg.H) + mk.shape)
    blocks = [0, cfg.nb // 2, cfg.nb - 1]
    rows = _rows(blocks, cfg.S)
    for h in (0, cfg.H - 1):
        rq, rk, rv = oracle.block_sparse_attention_bwd(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h]),
                                                       mk[0, h], 64, cfg.S_valid, q_blocks=blocks, kv_blocks=blocks)
        _check_head(f"dq[{h}]", dq[0, h], rq, rows)
        _check_head(f"dk[{h}]", dk[0, h], rk, rows)
        _check_head(f"dv[{h}]", dv[0, h], rv, rows)


def test_backward_order_tables_past_shared_memory(gpu_lib):
    """D = 64 with nb = 5460 key blocks in one head: the dQ kernel's shared buffer (8192 ints)
    cannot hold the longest-first order's tables (nb + 1 + ceil(nb/2) + 3 ints), so its
    workgroups keep the natural order; every gradient row is still written (NaN-initialised
    outputs) and sampled blocks match the oracle."""
    B, H, nb, D = 1, 1, 5460, 64
    S = nb * 64
    sv = S - 17
    g = torch.Generator(device="cpu").manual_seed(5)
    q, k, v, do = (torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(4))
    rng = np.random.default_rng(6)
    keep = np.zeros((nb, nb), bool)
    keep[np.arange(nb), np.arange(nb)] = True
    keep[np.arange(nb)[:, None], rng.integers(0, nb, size=(nb, 4))] = True
    m = torch.from_numpy(keep.astype(np.uint8)).to(DEV)
    o, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, m, s_valid=sv, return_lse=True)
    grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    dq, dk, dv = gpu_lib.block_sparse_attn_bwd(q, k, v, o, do, lse, m, s_valid=sv, out=grads)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(x).all(), name
    blocks = [0, 1, nb // 2, nb - 1]
    rows = _rows(blocks, S)
    rq, rk, rv = oracle.block_sparse_attention_bwd(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), f64(do[0, 0]), keep,
                                                   64, sv, q_blocks=blocks, kv_blocks=blocks)
    _check_head("dq", dq[0, 0], rq, rows)
    _check_head("dk", dk[0, 0], rk, rows)
    _check_head("dv", dv[0, 0], rv, rows)


def test_backward_deterministic(gpu_lib):
    q, k, v, do, m = _random_case(1, 2, 1024, 128, 1000, seed=11)
    a = _run(gpu_lib, q, k, v, do, m, 1000)
    b = _run(gpu_lib, q, k, v, do, m, 1000)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_plain_order_writes_every_row(gpu_lib):
    """14B shape with 3 heads (an odd head count, so items do not split evenly over the
    XCDs): its heads pair blocks one frame apart, so the backward kernels take their items in
    plain order. Every gradient row is written (NaN-initialised outputs, padded rows 0) and
    the result equals the gradients of the same heads computed one head at a time."""
    cfg = get_config(3, heads=3)
    q, k, v = make_inputs(cfg, seed=2, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(8)
    do = (torch.randn(q.shape, generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    m = gpu_lib.nabla_build_mask(q, k, cfg.thrs[0])
    rp, ci = gpu_lib.mask_to_csr(m)
    d = gpu_lib.attn_pair_offsets(q, rp, ci, s_valid=cfg.S_valid)
    assert int(d[0]) > 1, "this shape should pair blocks at an offset above 1"
    o, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, m, s_valid=cfg.S_valid, return_lse=True)
    grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    dq, dk, dv = gpu_lib.block_sparse_attn_bwd(q, k, v, o, do, lse, m, s_valid=cfg.S_valid, out=grads)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(x).all(), name
        assert torch.all(x[:, :, cfg.S_valid:] == 0), name
    for h in range(cfg.H):   # one head per call: a single-head launch
        sl = slice(h, h + 1)
        o1, l1 = gpu_lib.block_sparse_attn_fwd(q[:, sl], k[:, sl], v[:, sl], m[:, sl], s_valid=cfg.S_valid,
                                               return_lse=True)
        g1 = gpu_lib.block_sparse_attn_bwd(q[:, sl], k[:, sl], v[:, sl], o1, do[:, sl], l1, m[:, sl],
                                           s_valid=cfg.S_valid)
        torch.cuda.synchronize()
        for name, full, one in zip(("dq", "dk", "dv"), (dq, dk, dv), g1):
            assert torch.equal(full[:, sl], one), (name, h)
