"""Pins of the oracle's tiled decode (oracle/tiled.py) against what the diffusers PR page on Wan
tiling and the mathematics fix: the page's tile sizes, exact tiling of the video by the kept
regions, partition of unity of the blend, closed forms of the ramp on constant tiles, the
reductions to the untiled decode (one tile; no overlap). The page's figure for how far the
tiled decode moves from the untiled one (about 0.404, under its 0.5 assertion) belongs to
its test model's weights and is no pin here: the random-init tiny decoder on the page's CI
shape (128 x 128, tile 96, stride 64) moves by up to 1.68."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import round_bf16


def test_tile_grid_page_sizes():
    # defaults (tile 256, stride 192 video pixels) on the 704 x 1280 video's 44 x 80 latent
    assert oracle.tile_grid(44, 256, 192) == [(0, 16), (12, 16), (24, 16), (36, 8)]
    assert oracle.tile_grid(80, 256, 192) == [(0, 16), (12, 16), (24, 16), (36, 16), (48, 16), (60, 16), (72, 8)]
    # the page's CI case: a 128 x 128 video (8 x 8 latent), tile 96, stride 64
    assert oracle.tile_grid(8, 96, 64) == [(0, 6), (4, 4)]
    with pytest.raises(ValueError):
        oracle.tile_grid(8, 64, 96)
    with pytest.raises(ValueError):
        oracle.tile_grid(8, 100, 64)


@pytest.mark.parametrize("n", range(1, 30))
@pytest.mark.parametrize("tile,stride", [(256, 192), (96, 64), (64, 64), (48, 16), (32, 16)])
def test_kept_regions_tile_the_axis(n, tile, stride):
    """Brute force: the kept ranges [16 start, 16 start + min(stride, 16 size)) cover
    [0, 16 n) once each, in order, and every tile but the last is longer than the stride."""
    g = oracle.tile_grid(n, tile, stride)
    pos = 0
    for k, (i, sz) in enumerate(g):
        assert 16 * i == pos
        keep = min(stride, 16 * sz)
        if k < len(g) - 1:
            assert 16 * sz >= stride and keep == stride
        pos += keep
    assert pos == 16 * n


def _cut(img, gy, gx):
    return [[img[:, :, :, 16 * i:16 * (i + th), 16 * j:16 * (j + tw)].copy() for j, tw in gx] for i, th in gy]


@pytest.mark.parametrize("mode", ["fp64", "fp32", "bf16"])
@pytest.mark.parametrize("h,w,tile,stride", [(9, 13, (96, 128), (64, 64)), (8, 8, (96, 96), (64, 64)),
                                             (7, 5, (48, 48), (16, 32))])
def test_compose_is_a_partition_of_unity(mode, h, w, tile, stride):
    """Tiles cut from one image (integers in [-100, 100], exact in every mode; ramp weights
    with power-of-two E) compose back to that image exactly: the ramps are convex
    combinations of equal values, so any wrong row, column, offset or weight sum shows."""
    rng = np.random.default_rng(0)
    img = rng.integers(-100, 101, size=(2, 3, 2, 16 * h, 16 * w)).astype(np.float64)
    gy = oracle.tile_grid(h, tile[0], stride[0])
    gx = oracle.tile_grid(w, tile[1], stride[1])
    blend = (tile[0] - stride[0], tile[1] - stride[1])
    out = oracle.compose(_cut(img, gy, gx), stride, blend, mode)
    assert out.shape == img.shape
    assert np.array_equal(out, img)


def test_compose_ramp_closed_forms():
    """Constant tiles, fp64: two tiles one above the other, two side by side, and the corner
    of a 2 x 2 grid, against the ramp written out by hand."""
    E = 64
    H = W = 256

    def const(v, h=H, w=W):
        return np.full((1, 1, 1, h, w), float(v))

    A, B = 3.0, -5.0
    out = oracle.compose([[const(A)], [const(B)]], (192, 192), (E, E), "fp64")
    y = np.arange(E)
    # rows 192 + y of the video are the second tile's first E rows
    np.testing.assert_allclose(out[0, 0, 0, 192:192 + E, 7], A * (1 - y / E) + B * y / E, rtol=0, atol=1e-12)
    assert out[0, 0, 0, 191, 0] == A and out[0, 0, 0, 192 + E, 0] == B
    out = oracle.compose([[const(A), const(B)]], (192, 192), (E, E), "fp64")
    np.testing.assert_allclose(out[0, 0, 0, 5, 192:192 + E], A * (1 - y / E) + B * y / E, rtol=0, atol=1e-12)
    # 2 x 2: the corner (y, x < E) of tile (1, 1). Its vertical ramp meets tile (0, 1), whose
    # last rows carry that tile's own horizontal ramp with tile (0, 0); its horizontal ramp then
    # meets tile (1, 0), whose first rows carry that tile's vertical ramp with tile (0, 0).
    a00, a01, a10, a11 = 1.0, 2.0, 4.0, 8.0
    out = oracle.compose([[const(a00), const(a01)], [const(a10), const(a11)]], (192, 192), (E, E), "fp64")
    yy, xx = np.meshgrid(np.arange(E), np.arange(E), indexing="ij")
    v, u = yy / E, xx / E
    above = a00 * (1 - u) + a01 * u
    left = a00 * (1 - v) + a10 * v
    want = left * (1 - u) + (above * (1 - v) + a11 * v) * u
    np.testing.assert_allclose(out[0, 0, 0, 192:192 + E, 192:192 + E], want, rtol=0, atol=1e-12)


def test_compose_rounding_points_worked_value():
    """bf16, E = 3, tile above 1.0 and own tile -1.0, row 1: weights float32(2/3) and float32(1/3).
    1.0 x 0.6666667 rounds to bf16 0.66796875; -1.0 x 0.33333334 rounds to -0.333984375; their
    sum 0.333984375 is a bf16 value. Row 2: 0.33333334 -> 0.333984375 and -0.6666667 ->
    -0.66796875, sum -0.333984375. fp64 gives 1/3 and -1/3."""
    t = [[np.full((1, 1, 1, 64, 16), 1.0)], [np.full((1, 1, 1, 64, 16), -1.0)]]
    out = oracle.compose(t, (48, 16), (3, 0), "bf16")
    assert out[0, 0, 0, 48, 0] == 1.0
    assert out[0, 0, 0, 49, 0] == 0.333984375
    assert out[0, 0, 0, 50, 0] == -0.333984375
    assert out[0, 0, 0, 51, 0] == -1.0
    assert round_bf16(np.float32(2.0 / 3.0)) == 0.66796875
    out64 = oracle.compose(t, (48, 16), (3, 0), "fp64")
    assert abs(out64[0, 0, 0, 49, 0] - 1.0 / 3.0) < 1e-15


@pytest.fixture(scope="module")
def tiny():
    cfg = synthetic.DECODE_CONFIGS["tiny"]
    return cfg.latents(), cfg.weights()


def test_decode_tiled_one_tile_is_the_decode(tiny):
    z, W = tiny  # [1, 48, 2, 4, 4]: a 64 x 64 video
    assert np.array_equal(oracle.decode_tiled(z, W, "fp32", (64, 64), (64, 64)), oracle.decode(z, W, "fp32"))
    assert np.array_equal(oracle.decode_tiled(z, W, "fp32", (96, 80), (64, 64)), oracle.decode(z, W, "fp32"))


def test_decode_tiled_without_overlap_is_the_decode_of_each_crop(tiny):
    z, W = tiny
    out = oracle.decode_tiled(z, W, "fp32", (32, 32), (32, 32))
    for i in (0, 2):
        for j in (0, 2):
            crop = oracle.decode(np.ascontiguousarray(z[:, :, :, i:i + 2, j:j + 2]), W, "fp32")
            assert np.array_equal(out[:, :, :, 16 * i:16 * i + 32, 16 * j:16 * j + 32], crop)
