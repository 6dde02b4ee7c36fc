"""Pins for the sliding-tile mask oracle and the token layouts (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.sta import token_coords_of
from synth import token_coords


def _axis_pairs(n, r):
    # number of (a, c) pairs on one axis with |a - c| <= r, window cut at the border
    return sum(min(i + r, n - 1) - max(i - r, 0) + 1 for i in range(n))


@pytest.mark.parametrize("grid,tile,window,n_tile_pairs", [
    ((8, 32, 32), (4, 8, 8), (3, 3, 3), 400),        # 2 x 4 x 4 tiles
    ((30, 48, 80), (6, 8, 8), (3, 5, 5), 13728),     # 5 x 6 x 10 tiles
])
def test_tile_major_counts_closed_form(grid, tile, window, n_tile_pairs):
    G = [g // t for g, t in zip(grid, tile)]
    r = [w // 2 for w in window]
    closed = int(np.prod([_axis_pairs(g, rr) for g, rr in zip(G, r)]))
    assert closed == n_tile_pairs
    S = int(np.prod(grid))
    m = oracle.sta_block_mask(grid, "tile", tile, tile, window, 64, S)
    bpt = int(np.prod(tile)) // 64                                # blocks per tile
    assert m.sum() == n_tile_pairs * bpt * bpt
    assert np.array_equal(m, m.T)
    assert m.diagonal().all()


def test_aligned_equals_tile_mask_kron_ones():
    grid, tile, window = (8, 32, 32), (4, 8, 8), (3, 3, 3)
    m = oracle.sta_block_mask(grid, "tile", tile, tile, window, 64, 8192)
    G = [g // t for g, t in zip(grid, tile)]
    coords = np.stack(np.meshgrid(*[np.arange(g) for g in G], indexing="ij"), -1).reshape(-1, 3)
    tm = np.array([[all(abs(a[x] - c[x]) <= window[x] // 2 for x in range(3)) for c in coords]
                   for a in coords])
    assert np.array_equal(m, np.kron(tm, np.ones((4, 4), dtype=bool)))


def test_corner_tile_window_is_clipped():
    grid, tile, window = (30, 48, 80), (6, 8, 8), (3, 5, 5)
    m = oracle.sta_block_mask(grid, "tile", tile, tile, window, 64, 115200)
    # tile 0 sits in a corner: (1+1) * (2+1) * (2+1) visible tiles of 6 blocks
    assert m[0].sum() == 2 * 3 * 3 * 6


@pytest.mark.parametrize("grid,order,otile,tile,window", [
    ((3, 5, 6), "row", None, (2, 2, 3), (3, 3, 3)),
    ((4, 4, 8), "tile", (2, 2, 4), (2, 2, 4), (1, 3, 3)),
    ((5, 3, 7), "row", None, (2, 2, 2), (3, 1, 5)),
])
def test_any_pair_rule_brute_force(grid, order, otile, tile, window):
    """Block mask = OR over token pairs of the token-level window rule, by loops."""
    n = 8
    coords = token_coords_of(grid, order, otile)
    Sv = len(coords)
    S = -(-Sv // n) * n
    r = [w // 2 for w in window]
    nb = S // n
    expect = np.zeros((nb, nb), dtype=bool)
    for p in range(Sv):
        for q in range(Sv):
            a = [coords[p][x] // tile[x] for x in range(3)]
            c = [coords[q][x] // tile[x] for x in range(3)]
            if all(abs(a[x] - c[x]) <= r[x] for x in range(3)):
                expect[p // n, q // n] = True
    got = oracle.sta_block_mask(grid, order, otile, tile, window, n, S)
    assert np.array_equal(got, expect)
    tok = oracle.sta_token_mask(grid, order, otile, tile, window)
    assert tok.shape == (Sv, Sv)


@pytest.mark.parametrize("grid,order,tile", [
    ((4, 8, 8), "row", None), ((8, 32, 32), "tile", (4, 8, 8)), ((30, 48, 80), "tile", (6, 8, 8)),
    ((21, 45, 80), "row", None), ((5, 6, 7), "tile", (2, 4, 4)),
])
def test_layouts_agree_with_generator(grid, order, tile):
    a = token_coords_of(grid, order, tile)
    b = token_coords(grid, order, tile)
    assert np.array_equal(a, b)
    assert len(np.unique(a, axis=0)) == np.prod(grid)       # a permutation of the grid


def test_config5_fraction():
    m = oracle.sta_block_mask((21, 45, 80), "row", None, (4, 8, 8), (3, 3, 3), 64, 75648)
    assert m.shape == (1182, 1182)
    assert np.array_equal(m, m.T) and m.diagonal().all()
    assert 0.2 < m.mean() < 0.3
