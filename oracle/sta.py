"""Static sliding-tile (STA-style) block mask (test infrastructure only).

Source: the blog review "Fast Video Generation with SLIDING TILE ATTENTION",
section "Observation & Proposed Method", and the STA abstract in the Daily Papers
listing: tokens are grouped into 3D tiles; all queries of one tile attend to the
same keys, those of the tiles inside a local 3D window around the query tile; with
the tile equal to the attention block there are no partially used blocks.

Readings (listed in the design notes):
  * the window is centred on the query tile, w tiles wide along each axis, so key
    tile c is visible from query tile a iff |a - c| <= floor(w / 2) per axis; at the
    grid border the window is cut off, not shifted;
  * grids that tiles do not divide get smaller border tiles;
  * an N-token block pair (i, j) is kept iff some real token of block i and some
    real token of block j are allowed (any-pair rule); blocks are computed whole.
"""
import numpy as np


def token_coords_of(grid, order, order_tile=None) -> np.ndarray:
    """(t, h, w) of each sequence position, by explicit enumeration."""
    T, H, W = grid
    out = []
    if order == "row":
        for t in range(T):
            for h in range(H):
                for w in range(W):
                    out.append((t, h, w))
    elif order == "tile":
        tt, th, tw = order_tile
        for a in range(-(-T // tt)):
            for b in range(-(-H // th)):
                for c in range(-(-W // tw)):
                    for t in range(a * tt, min(T, (a + 1) * tt)):
                        for h in range(b * th, min(H, (b + 1) * th)):
                            for w in range(c * tw, min(W, (c + 1) * tw)):
                                out.append((t, h, w))
    else:
        raise ValueError(order)
    return np.array(out, dtype=np.int64)


def _tile_ids(grid, tile, coords):
    G = [-(-g // s) for g, s in zip(grid, tile)]
    tc = coords // np.asarray(tile)
    return (tc[:, 0] * G[1] + tc[:, 1]) * G[2] + tc[:, 2], G


def _near(G, window):
    """Near[a, c] = key tile c lies in the window of query tile a."""
    r = np.asarray(window) // 2
    a = np.stack(np.meshgrid(*[np.arange(g) for g in G], indexing="ij"), -1).reshape(-1, 3)
    diff = np.abs(a[:, None, :] - a[None, :, :])
    return np.all(diff <= r, axis=-1)


def sta_token_mask(grid, order, order_tile, tile, window) -> np.ndarray:
    """Token-level mask [S_v, S_v]: query token p may see key token q."""
    coords = token_coords_of(grid, order, order_tile)
    tid, G = _tile_ids(grid, tile, coords)
    near = _near(G, window)
    return near[tid[:, None], tid[None, :]]


def sta_block_mask(grid, order, order_tile, tile, window, n: int, S: int) -> np.ndarray:
    """Block mask [S/n, S/n] under the any-pair rule.

    With Occ[i, a] = "block i holds a real token of tile a" and Near as above, the
    block pair (i, j) is kept iff sum_{a,c} Occ[i,a] Near[a,c] Occ[j,c] > 0.
    """
    coords = token_coords_of(grid, order, order_tile)
    tid, G = _tile_ids(grid, tile, coords)
    nb = S // n
    n_tiles = int(np.prod(G))
    occ = np.zeros((nb, n_tiles), dtype=np.int64)
    occ[np.arange(len(tid)) // n, tid] = 1
    near = _near(G, window).astype(np.int64)
    return (occ @ near @ occ.T) > 0
