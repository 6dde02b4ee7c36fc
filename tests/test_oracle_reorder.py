"""Pins for the token reordering of the oracle (CPU only)."""
import numpy as np
import pytest

from oracle.reorder import order_coords, reorder_tokens


@pytest.mark.parametrize("grid,order,tile", [((4, 8, 8), "tile", (1, 4, 4)), ((5, 6, 7), "tile", (2, 4, 3)),
                                             ((3, 5, 4), "spatial", None), ((2, 3, 3), "row", None)])
def test_orders_are_permutations_and_round_trip(grid, order, tile):
    S_valid = int(np.prod(grid))
    S = -(-S_valid // 64) * 64
    x = np.random.default_rng(0).standard_normal((2, S, 5))
    y = reorder_tokens(x, grid, order, tile)
    assert np.all(y[:, S_valid:] == 0)
    assert sorted(map(tuple, order_coords(grid, order, tile))) == sorted(
        (t, h, w) for t in range(grid[0]) for h in range(grid[1]) for w in range(grid[2]))
    back = reorder_tokens(y, grid, order, tile, inverse=True)
    assert np.array_equal(back[:, :S_valid], x[:, :S_valid]) and np.all(back[:, S_valid:] == 0)


def test_fractal_flattening_blocks_are_frame_patches():
    # tile 1 x P x P with P = 8 on a 3 x 16 x 24 grid: every 64-token block is one frame's 8 x 8 patch
    T, H, W, P = 3, 16, 24, 8
    c = order_coords((T, H, W), "tile", (1, P, P))
    for blk in range(T * H * W // 64):
        cc = c[blk * 64:(blk + 1) * 64]
        assert len(set(cc[:, 0])) == 1
        assert cc[:, 1].max() - cc[:, 1].min() == P - 1 and cc[:, 2].max() - cc[:, 2].min() == P - 1
        assert cc[0, 1] % P == 0 and cc[0, 2] % P == 0
    # the patches of a frame in row-major patch order, frames in order
    firsts = c[::64]
    assert [tuple(f) for f in firsts[:4]] == [(0, 0, 0), (0, 0, 8), (0, 0, 16), (0, 8, 0)]


def test_spatial_order_closed_form():
    T, H, W = 4, 3, 5
    c = order_coords((T, H, W), "spatial")
    p = np.arange(T * H * W)
    assert np.array_equal(c[:, 0], p % T)
    assert np.array_equal(c[:, 1] * W + c[:, 2], p // T)
