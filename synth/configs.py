"""The five workloads: shapes, dtypes, thresholds and sliding-tile specs.

Each entry is a video-DiT self-attention shape: a T x H x W latent grid flattened
into one token sequence, cut into N = 64 token blocks.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class StaSpec:
    """A static sliding-tile mask: tokens grouped in tiles, each query tile sees a
    window of whole tiles around it (clipped at the grid border)."""
    tile: Tuple[int, int, int]      # tokens per tile along (t, h, w)
    window: Tuple[int, int, int]    # window size in tiles along (t, h, w), odd


@dataclass(frozen=True)
class Config:
    cid: int                        # stable id, part of every seed
    name: str
    B: int
    H: int
    D: int
    grid: Tuple[int, int, int]      # latent (T, H, W)
    order: str                      # "row" (t,h,w row-major) or "tile" (tile-major)
    order_tile: Optional[Tuple[int, int, int]]  # tile used by the tile-major order
    dtype: str                      # "f32" or "bf16"
    sigma: float                    # std of the i.i.d. noise part
    pos_amp: float                  # amplitude of each positional sinusoid (0 = none)
    thrs: Tuple[float, ...]         # NABLA thresholds (empty = no adaptive mask)
    sta: Optional[StaSpec]          # sliding-tile mask OR'd in (None = none)
    fp8_run: bool = False           # also run with fp8 e4m3 Q/K and per-block scales
    dense_timing: bool = False      # also time the all-ones mask
    N: int = 64

    @property
    def S_valid(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def S(self) -> int:
        return -(-self.S_valid // self.N) * self.N

    @property
    def nb(self) -> int:
        return self.S // self.N


CONFIGS = {
    1: Config(1, "tiny-4x8x8", B=1, H=2, D=64, grid=(4, 8, 8), order="row", order_tile=None,
              dtype="f32", sigma=1.0, pos_amp=1.0, thrs=(0.2,), sta=None),
    2: Config(2, "dit2b-8x32x32", B=1, H=16, D=128, grid=(8, 32, 32), order="tile",
              order_tile=(4, 8, 8), dtype="bf16", sigma=0.5, pos_amp=1.0, thrs=(0.1,),
              sta=StaSpec(tile=(4, 8, 8), window=(3, 3, 3))),
    3: Config(3, "t2v14b-21x45x80", B=1, H=40, D=128, grid=(21, 45, 80), order="row",
              order_tile=None, dtype="bf16", sigma=1.0, pos_amp=1.0, thrs=(0.2,), sta=None,
              dense_timing=True),
    4: Config(4, "hunyuan-30x48x80", B=1, H=24, D=128, grid=(30, 48, 80), order="tile",
              order_tile=(6, 8, 8), dtype="bf16", sigma=1.0, pos_amp=0.0, thrs=(),
              sta=StaSpec(tile=(6, 8, 8), window=(3, 5, 5))),
    5: Config(5, "sweep-21x45x80", B=1, H=40, D=128, grid=(21, 45, 80), order="row",
              order_tile=None, dtype="bf16", sigma=1.0, pos_amp=1.0,
              thrs=(0.05, 0.1, 0.2, 0.4), sta=StaSpec(tile=(4, 8, 8), window=(3, 3, 3)),
              fp8_run=True),
}


def get_config(i: int, heads: Optional[int] = None) -> Config:
    """Config i, optionally with fewer heads (same per-head shape) for quick checks."""
    c = CONFIGS[i]
    if heads is not None and heads != c.H:
        from dataclasses import replace
        c = replace(c, H=heads, name=f"{c.name}-h{heads}")
    return c
