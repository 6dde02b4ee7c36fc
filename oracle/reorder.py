"""Token reordering between the row-major (t, h, w) layout and the mask-friendly
layouts (test infrastructure only).

Sources: NABLA (Pith review, "Assumptions & free parameters" and Figure 4): fractal
flattening groups each frame into P x P spatial patches; STA blog review ("Observation
& Proposed Method"): tokens grouped into 3D tiles; SVG (blog review of Sparse VideoGen):
a layout transformation that puts the tokens of one spatial position across frames
together. Readings (design notes): "tile" = tiles row-major, tokens row-major inside a
tile (fractal flattening is tile 1 x P x P); "spatial" = (h, w, t) order. The sequence
is padded with zero rows after the T*H*W tokens.
"""
import numpy as np

from .sta import token_coords_of


def order_coords(grid, order, tile=None) -> np.ndarray:
    """(t, h, w) of every position of the order, by explicit enumeration."""
    T, H, W = grid
    if order in ("row", "tile"):
        return token_coords_of(grid, order, tile)
    if order == "spatial":
        return np.array([(t, h, w) for h in range(H) for w in range(W) for t in range(T)], dtype=np.int64)
    raise ValueError(order)


def reorder_tokens(x, grid, order, tile=None, inverse=False):
    """x [..., S, D] -> same shape. inverse=False: row-major -> `order`; True: back.
    Rows >= T*H*W of the result are 0."""
    x = np.asarray(x)
    T, H, W = grid
    c = order_coords(grid, order, tile)
    rowmajor = (c[:, 0] * H + c[:, 1]) * W + c[:, 2]       # position p of the order holds token rowmajor[p]
    n = len(rowmajor)
    out = np.zeros_like(x)
    if inverse:
        out[..., rowmajor, :] = x[..., :n, :]
    else:
        out[..., :n, :] = x[..., rowmajor, :]
    return out
