"""GPU parity of token reordering (bit for bit: pure data movement) against the oracle."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("grid,order,tile,dtype,D", [
    ((8, 32, 32), "tile", (4, 8, 8), torch.bfloat16, 128),        # 2B-DiT layout, aligned tiles
    ((21, 45, 80), "tile", (4, 8, 8), torch.bfloat16, 128),       # 14B grid, ragged border tiles, end padding
    ((5, 24, 40), "tile", (1, 8, 8), torch.float32, 64),          # fractal flattening, P = 8
    ((7, 9, 11), "spatial", None, torch.bfloat16, 64),
    ((6, 10, 10), "tile", (3, 4, 6), torch.uint8, 128),           # fp8 codes, 128-byte rows
    ((4, 4, 4), "row", None, torch.bfloat16, 128),
])
def test_reorder_matches_oracle_and_round_trips(gpu_lib, grid, order, tile, dtype, D):
    S_valid = int(np.prod(grid))
    S = -(-S_valid // 64) * 64
    g = torch.Generator(device="cpu").manual_seed(S_valid)
    if dtype == torch.uint8:
        x = torch.randint(0, 256, (2, 3, S, D), generator=g, dtype=torch.uint8)
    else:
        x = torch.randn(2, 3, S, D, generator=g).to(dtype)
    x = x.to(DEV)
    print(f"[reorder] grid {grid} order {order} tile {tile} {dtype} D {D}", flush=True)
    y = gpu_lib.token_reorder(x, grid, order, tile)
    back = gpu_lib.token_reorder(y, grid, order, tile, inverse=True)
    torch.cuda.synchronize()
    xc = x.cpu()
    xn = xc.view(torch.int16).numpy() if dtype == torch.bfloat16 else xc.numpy()
    ref = oracle.reorder_tokens(xn, grid, order, tile)
    yn = y.cpu().view(torch.int16).numpy() if dtype == torch.bfloat16 else y.cpu().numpy()
    assert np.array_equal(yn, ref)
    bn = back.cpu().view(torch.int16).numpy() if dtype == torch.bfloat16 else back.cpu().numpy()
    assert np.array_equal(bn, oracle.reorder_tokens(ref, grid, order, tile, inverse=True))
    assert np.array_equal(bn[..., :S_valid, :], xn[..., :S_valid, :])


def test_reorder_strided_views(gpu_lib):
    grid, tile = (4, 16, 16), (2, 8, 8)
    big = torch.randn(1, 6, 1024, 256, generator=torch.Generator(device="cpu").manual_seed(1)).to(torch.bfloat16)
    x = big.to(DEV)[:, 1:4, :, 128:]                                # head and row strides of the parent
    out = torch.zeros(1, 3, 1024, 128, dtype=torch.bfloat16, device=DEV)
    gpu_lib.token_reorder(x, grid, "tile", tile, out=out)
    torch.cuda.synchronize()
    ref = oracle.reorder_tokens(x.cpu().view(torch.int16).numpy(), grid, "tile", tile)
    assert np.array_equal(out.cpu().view(torch.int16).numpy(), ref)
