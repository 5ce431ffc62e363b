"""Spatially tiled decode (test infrastructure, like the rest of ``oracle/``).

Page 4 (diffusers PR "Implement tiled VAE encoding/decoding for Wan model") adds an opt-in
tiled decode to diffusers' Wan VAE: the latent is cut into overlapping spatial tiles, each
tile is decoded on its own, and the decoded tiles are blended where they overlap. The page
gives the tile size and stride (256 and 192 video pixels by default; its CI test uses a
128 x 128 video with tile 96 and stride 64) and the size of the difference this makes
(about 0.404 at most against the untiled decode there, under its 0.5 assertion). It does
not state the blend rule. The reading taken here, the one diffusers' VAEs use:

* Tiles along each axis start at latent 0, s, 2s, ... below the latent size, s = stride / 16,
  and cover t = tile / 16 latents or what is left (16 video pixels per latent pixel: the
  decoder's 8x and unpatchify's 2x).
* Each tile is decoded as a video of its own (``decode``: its own causal caches, unpatchify,
  clamp).
* The tiles are then composed in raster order. A tile first takes a linear ramp with the
  tile above over its first E_v = min(H_above, H, tile - stride) rows: row y becomes
  above[H_above - E_v + y] * (1 - y / E_v) + own[y] * (y / E_v). Then it takes the same ramp
  with the tile to its left over its first E_h columns. The neighbours enter as already
  composed (their own ramps applied).
* The output keeps rows [0, stride) and columns [0, stride) of every composed tile, which
  tile the video exactly.
* In fp32 and bf16 each product and the sum round to the storage type, the weights being
  float32 constants (elementwise tensor arithmetic in that dtype).
"""
from __future__ import annotations

import numpy as np

from .decoder import Prec, decode

SPATIAL = 16  # video pixels per latent pixel


def tile_grid(n_latent: int, tile_px: int, stride_px: int) -> list[tuple[int, int]]:
    """(start, size) in latent units of the tiles along one axis of n_latent latents."""
    if tile_px % SPATIAL or stride_px % SPATIAL or not 0 < stride_px <= tile_px:
        raise ValueError(f"tile {tile_px} and stride {stride_px} must be multiples of {SPATIAL}, "
                         "0 < stride <= tile")
    t, s = tile_px // SPATIAL, stride_px // SPATIAL
    return [(i, min(t, n_latent - i)) for i in range(0, n_latent, s)]


def _ramp(P: Prec, other, own, E: int, axis: int) -> np.ndarray:
    """own's first E entries along ``axis`` blended with other's last E there (see the module
    docstring); own is modified in place and returned."""
    for y in range(E):
        wo = P.scalar(1.0 - y / E)
        wn = P.scalar(y / E)
        a = np.take(other, other.shape[axis] - E + y, axis=axis)
        idx = [slice(None)] * own.ndim
        idx[axis] = y
        b = own[tuple(idx)]
        own[tuple(idx)] = P.R(P.R(a * wo) + P.R(b * wn))
    return own


def compose(tiles, stride_px: tuple[int, int], blend_px: tuple[int, int], mode: str = "fp32") -> np.ndarray:
    """tiles[r][c]: the decoded tile videos [B, 3, F, H_rc, W_rc] of one tile grid. Returns the
    composed video [B, 3, F, sum of kept rows, sum of kept columns]."""
    P = Prec(mode)
    sy, sx = stride_px
    done = [[None] * len(row) for row in tiles]
    for r, row in enumerate(tiles):
        for c, t in enumerate(row):
            own = np.array(t, dtype=P.store, copy=True)
            if r > 0:
                above = done[r - 1][c]
                E = min(above.shape[3], own.shape[3], blend_px[0])
                _ramp(P, above, own, E, 3)
            if c > 0:
                left = done[r][c - 1]
                E = min(left.shape[4], own.shape[4], blend_px[1])
                _ramp(P, left, own, E, 4)
            done[r][c] = own
    rows = [np.concatenate([t[:, :, :, :sy, :sx] for t in row], axis=4) for row in done]
    return np.concatenate(rows, axis=3)


def decode_tiled(z, weights, mode: str = "fp32", tile_px=(256, 256), stride_px=(192, 192),
                 acc: str = "f64") -> np.ndarray:
    """The tiled decode of latents z [B, 48, T, h, w] -> video [B, 3, 4T-3, 16h, 16w]: every
    tile of the grid decoded with ``decode``, then composed."""
    gy = tile_grid(z.shape[3], tile_px[0], stride_px[0])
    gx = tile_grid(z.shape[4], tile_px[1], stride_px[1])
    tiles = [[decode(np.ascontiguousarray(z[:, :, :, i:i + th, j:j + tw]), weights, mode, acc) for j, tw in gx]
             for i, th in gy]
    blend = (tile_px[0] - stride_px[0], tile_px[1] - stride_px[1])
    return compose(tiles, stride_px, blend, mode)
