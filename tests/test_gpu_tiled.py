"""Parity of wanvae_decode_tiled (the spatially tiled decode of the diffusers PR page on Wan
tiling) with the oracle's tiled decode (oracle/tiled.py): fp32 max 5e-4; bf16 PSNR >= 40 dB
and within the oracle's own bf16-vs-fp32 distance (gate_bf16_scale: every tile is a
multi-chunk decode of the tiny decoder; measured 0.0036 mean against 0.0043 there, while the
oracle's float32-sum variant moves by only 0.0013 on one of the cases). The reductions to
the untiled decode (one tile, no overlap) hold on the GPU too, and at the 704 x 1280 size
the composition of the tiles is checked against the oracle's composition of the same
decoded tiles."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import TORCH, dev, gate_bf16_scale, say, to_np
from video_vae_decoding_amd import wanvae

pytestmark = pytest.mark.gpu


def to_gpu(z, W):
    return torch.from_numpy(z).to(dev()), {k: torch.from_numpy(v).to(dev()) for k, v in W.items()}


def gpu_tiled(z, W, mode, tile, stride):
    zt, Wt = to_gpu(z, W)
    v = wanvae.wanvae_decode_tiled(zt, Wt, TORCH[mode], tile, stride)
    torch.cuda.synchronize()
    return v


CASES = [  # (latent [B, 48, T, h, w], tile, stride)
    ((2, 48, 3, 8, 10), (96, 96), (64, 64)),  # the page's CI tile and stride; widths 6, 6, 2 latents
    ((1, 48, 2, 7, 9), (64, 96), (32, 48)),   # ragged rows (4, 4, 3, 1) and columns (6, 6, 3)
]


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
@pytest.mark.parametrize("shape,tile,stride", CASES)
def test_tiled_decode_matches_oracle(mode, shape, tile, stride):
    z = synthetic.normal(12, "latents_tiled", shape)
    W = synthetic.gen_weights(16, 12, 0.1)
    say("tiled decode", shape, tile, stride, mode)
    got = to_np(gpu_tiled(z, W, mode, tile, stride))
    want = oracle.decode_tiled(z, W, mode, tile, stride)
    assert got.shape == want.shape == (shape[0], 3, 4 * shape[2] - 3, 16 * shape[3], 16 * shape[4])
    d = np.abs(got.astype(np.float64) - want)
    p = oracle.psnr(got, want)
    if mode == "fp32":
        say("max", d.max(), "psnr", p)
        assert d.max() <= 5e-4, d.max()
        return
    gate_bf16_scale(got, want, oracle.decode_tiled(z, W, "fp32", tile, stride).astype(np.float64),
                    f"tiled {shape} bf16")


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_one_tile_is_the_decode_bit_for_bit(mode):
    cfg = synthetic.DECODE_CONFIGS["tiny"]
    z, W = cfg.latents(), cfg.weights()
    zt, Wt = to_gpu(z, W)
    tiled = wanvae.wanvae_decode_tiled(zt, Wt, TORCH[mode], (64, 96), (64, 64))
    plain = wanvae.wanvae_decode(zt, Wt, TORCH[mode])
    torch.cuda.synchronize()
    assert torch.equal(tiled, plain)


def test_no_overlap_fp32_is_the_decode_of_each_crop():
    """stride = tile: no ramp; every tile's block is the decode of its latent crop (fp32: the
    kernels' sums do not depend on the batch the tile shares)."""
    z = synthetic.normal(13, "latents_tiled", (1, 48, 2, 6, 5))
    W = synthetic.gen_weights(16, 13, 0.1)
    zt, Wt = to_gpu(z, W)
    tiled = to_np(wanvae.wanvae_decode_tiled(zt, Wt, torch.float32, (48, 32), (48, 32)))
    for i in (0, 3):
        for j in (0, 2, 4):
            crop = zt[:, :, :, i:i + 3, j:j + 2].contiguous()
            want = to_np(wanvae.wanvae_decode(crop, Wt, torch.float32))
            torch.cuda.synchronize()
            got = tiled[:, :, :, 16 * i:16 * i + 16 * crop.shape[3], 16 * j:16 * j + 16 * crop.shape[4]]
            assert np.abs(got.astype(np.float64) - want).max() <= 1e-6


def test_full_size_composition_matches_the_oracle_composition():
    """704 x 1280 (44 x 80 latent), bf16, the page's default tile 256 / stride 192, 3 latent
    frames: the library's tiled decode against oracle.compose of the same decoded tiles, got
    from wanvae_decode on each tile row's equal-width batch (the same decodes the tiled entry
    runs), bit for bit."""
    cfg = synthetic.DECODE_CONFIGS["ti2v5b_landscape"]
    z = np.ascontiguousarray(cfg.latents()[:, :, :3])
    W = cfg.weights()
    tile, stride = (256, 256), (192, 192)
    say("full-size tiled decode, 3 latent frames")
    zt, Wt = to_gpu(z, W)
    got = wanvae.wanvae_decode_tiled(zt, Wt, torch.bfloat16, tile, stride)
    torch.cuda.synchronize()
    gy, gx = oracle.tile_grid(cfg.h, 256, 192), oracle.tile_grid(cfg.w, 256, 192)
    tiles = []
    for i, th in gy:
        row = [None] * len(gx)
        widths = sorted({tw for _, tw in gx}, reverse=True)
        for tw in widths:
            cols = [c for c, (_, w_) in enumerate(gx) if w_ == tw]
            batch = torch.cat([zt[:, :, :, i:i + th, gx[c][0]:gx[c][0] + tw] for c in cols], 0).contiguous()
            v = wanvae.wanvae_decode(batch, Wt, torch.bfloat16)
            torch.cuda.synchronize()
            for k, c in enumerate(cols):
                row[c] = to_np(v[k:k + 1]).astype(np.float32)
        tiles.append(row)
    say("composing on the CPU")
    want = oracle.compose(tiles, stride, (64, 64), "bf16")
    assert want.shape == tuple(got.shape)
    assert np.array_equal(to_np(got).astype(np.float32), want)
    assert torch.isfinite(got).all()
    del got
    torch.cuda.empty_cache()
