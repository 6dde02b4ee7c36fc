"""Seeded generator for Q, K, V shaped like video-DiT self-attention.

Recipe (per batch b, head h):
  * tokens are the cells (t, h, w) of the latent grid, placed in the sequence in
    the config's order (row-major, or tile-major with row-major tokens inside a
    tile); the sequence is zero-padded at the end to a multiple of N;
  * a smooth positional term P[pos, d] = A * sum_{m<8} sin(wt*t + wh*h + ww*w + phi)
    with wt, wh, ww ~ U(0, 0.5) rad per grid step and phi ~ U(0, 2 pi), drawn per
    (head, channel, m); the same P is added to Q and K, never to V;
  * Q = sigma*eps_q + P, K = sigma*eps_k + P, V = sigma*eps_v with eps ~ N(0, 1);
  * the result is rounded to the config dtype (bf16 round-to-nearest-even, or f32).
Every draw comes from a torch.Generator seeded by (config id, b, h, tensor, seed),
so a given device always produces the same tensors.
"""
import zlib
from typing import Optional, Tuple

import numpy as np
import torch

from .configs import Config

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def token_coords(grid: Tuple[int, int, int], order: str,
                 tile: Optional[Tuple[int, int, int]] = None) -> np.ndarray:
    """(t, h, w) of every sequence position, int64 [T*H*W, 3]."""
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    rm = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)   # row-major order
    if order == "row":
        return rm
    if order != "tile":
        raise ValueError(f"unknown token order {order!r}")
    tt, th, tw = tile
    # tile-major: sort by (tile index row-major, then row-major position inside the tile)
    tiles_h = -(-H // th)
    tiles_w = -(-W // tw)
    tid = ((rm[:, 0] // tt) * tiles_h + rm[:, 1] // th) * tiles_w + rm[:, 2] // tw
    inner = ((rm[:, 0] % tt) * th + rm[:, 1] % th) * tw + rm[:, 2] % tw
    perm = np.lexsort((inner, tid))
    return rm[perm]


def _seed(cfg: Config, b: int, h: int, tensor: int, seed: int) -> int:
    key = f"{cfg.cid}/{b}/{h}/{tensor}/{seed}".encode()
    return zlib.crc32(key) & 0x7FFFFFFF


def _positional(coords: torch.Tensor, D: int, gen: torch.Generator, amp: float) -> torch.Tensor:
    dev = coords.device
    omega = torch.rand(D, 8, 3, generator=gen, device=dev) * 0.5
    phi = torch.rand(D, 8, generator=gen, device=dev) * (2 * np.pi)
    c = coords.to(torch.float32)                                    # [S_v, 3]
    out = torch.zeros(c.shape[0], D, device=dev, dtype=torch.float32)
    for m in range(8):
        arg = c @ omega[:, m, :].T + phi[:, m]                      # [S_v, D]
        out += torch.sin(arg)
    return out * amp


def make_inputs(cfg: Config, seed: int = 0, device="cpu"):
    """Q, K, V as [B, H, S, D] tensors of the config dtype on `device`."""
    dev = torch.device(device)
    dt = _DT[cfg.dtype]
    B, H, S, D, Sv = cfg.B, cfg.H, cfg.S, cfg.D, cfg.S_valid
    coords = torch.from_numpy(token_coords(cfg.grid, cfg.order, cfg.order_tile)).to(dev)
    q = torch.zeros(B, H, S, D, dtype=dt, device=dev)
    k = torch.zeros(B, H, S, D, dtype=dt, device=dev)
    v = torch.zeros(B, H, S, D, dtype=dt, device=dev)
    for b in range(B):
        for h in range(H):
            gp = torch.Generator(device=dev)
            gp.manual_seed(_seed(cfg, b, h, 3, seed))
            pos = _positional(coords, D, gp, cfg.pos_amp) if cfg.pos_amp else None
            for ti, dst in enumerate((q, k, v)):
                g = torch.Generator(device=dev)
                g.manual_seed(_seed(cfg, b, h, ti, seed))
                x = torch.randn(Sv, D, generator=g, device=dev) * cfg.sigma
                if pos is not None and ti < 2:
                    x += pos
                dst[b, h, :Sv] = x.to(dt)
    return q, k, v


def make_signs(D: int, seed: int = 0):
    """D random signs (+1.0 / -1.0, float64 numpy array) from a seeded torch generator: the
    random draw of the incoherent processing, passed to both the library and the oracle."""
    g = torch.Generator()
    g.manual_seed(0x5167 + seed)
    bits = torch.randint(0, 2, (D,), generator=g)
    return (1.0 - 2.0 * bits.double()).numpy()


def quantize_fp8_blocks(x: torch.Tensor, N: int = 64):
    """Per (b, h, N-token block) fp8 e4m3fn quantization with scale = amax / 448.

    Returns (codes as uint8 [B,H,S,D], scales float32 [B,H,S/N]). Decoding a code c
    of block j gives fp8(c) * scale[j]. All-zero blocks get scale 1.
    """
    B, H, S, D = x.shape
    xf = x.to(torch.float32).reshape(B, H, S // N, N, D)
    amax = xf.abs().amax(dim=(3, 4))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (xf / scale[..., None, None]).to(torch.float8_e4m3fn)
    return q.reshape(B, H, S, D).view(torch.uint8), scale.contiguous()
