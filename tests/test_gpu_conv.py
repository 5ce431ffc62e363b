"""Parity of wanvae_causal_conv3d (one causal conv with its cached history) with the oracle.

Small ragged shapes (several tiles, partial tiles in channels, positions and K) are compared
element by element; the two full-size convs on sampled outputs, each an oracle dot product.
fp32: |gpu - oracle| within the probabilistic float32 summation bound 8 sqrt(K) 2^-24 sum|w x|.
bf16: within one bf16 spacing of the oracle's rounded result plus that bound (the float32 sums
before the rounding may differ by it), almost all bit-equal.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import acc_bound, assert_bf16_close, dev, rounded, say, to_dev, to_np
from video_vae_decoding_amd import wanvae

pytestmark = pytest.mark.gpu

# (Cin, Cout, kt, kh, kw, t, h, w, n_cache, B)
SMALL = [
    (40, 20, 3, 3, 3, 3, 5, 7, 2, 2),
    (136, 144, 3, 3, 3, 2, 9, 30, 1, 1),
    (64, 32, 3, 1, 1, 4, 6, 6, 0, 1),
    (48, 48, 1, 1, 1, 3, 4, 5, 0, 2),
    (32, 64, 1, 3, 3, 2, 7, 5, 0, 1),
    (256, 12, 3, 3, 3, 4, 8, 8, 2, 1),
    (64, 256, 3, 3, 3, 1, 3, 50, 2, 1),
]


# bf16 convs the halo-tile kernel takes by default (3x3, Cin % 32 == 0, Cout % 128 == 0, frames
# of at least 32 x 64, at least 16,384 positions): ragged 16 x 32 blocks, batch 2, a 2-D conv,
# and a 62 x 80 frame, which 32 x 16 blocks pad less than 16 x 32 ones (64 x 80 against 64 x 96)
HALO = [
    (32, 128, 3, 3, 3, 2, 40, 210, 2, 2),
    (64, 256, 1, 3, 3, 1, 70, 120, 0, 2),
    (32, 128, 3, 3, 3, 2, 62, 80, 2, 2),
]


def run_gpu(x, cache, w, b, mode, layout):
    xt, wt, bt = to_dev(x, mode), to_dev(w, mode), to_dev(b, mode)
    ct = to_dev(cache, mode) if cache is not None and cache.shape[2] else None
    if layout == "nthwc":
        xt = xt.permute(0, 2, 3, 4, 1).contiguous()
        ct = ct.permute(0, 2, 3, 4, 1).contiguous() if ct is not None else None
    y = wanvae.wanvae_causal_conv3d(xt, ct, wt, bt, layout=layout)
    torch.cuda.synchronize()
    y = to_np(y)
    return y.transpose(0, 4, 1, 2, 3) if layout == "nthwc" else y


def check(got, x, cache, w, b, mode, what):
    P = oracle.Prec(mode)
    xr, cr, wr, br = (rounded(a, mode) if a is not None else None for a in (x, cache, w, b))
    hist = cr if cr is not None and cr.shape[2] else None
    want = oracle.causal_conv(xr, wr, br, hist, P)
    mag = oracle.causal_conv(np.abs(xr), np.abs(wr), np.abs(br), None if hist is None else np.abs(hist), oracle.Prec("fp64"))
    err = acc_bound(w[0].size, mag)
    if mode == "fp32":
        d = np.abs(got.astype(np.float64) - want)
        assert np.all(d <= err + 2.0 ** -24 * np.abs(want)), f"{what}: max diff {d.max():.3g}"
        assert d.max() <= 1e-3
    else:
        assert_bf16_close(got, want, err, what=what)


def inputs(case):
    Ci, Co, kt, kh, kw, t, h, w, nc, B = case
    g = np.random.default_rng(abs(hash(case)) % 2**31)
    x = g.standard_normal((B, Ci, t, h, w)).astype(np.float32)
    cache = g.standard_normal((B, Ci, nc, h, w)).astype(np.float32) if nc else None
    wgt = (g.standard_normal((Co, Ci, kt, kh, kw)) / np.sqrt(Ci * kt * kh * kw)).astype(np.float32)
    b = (0.1 * g.standard_normal(Co)).astype(np.float32)
    return x, cache, wgt, b


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", ["ncthw", "nthwc"])
@pytest.mark.parametrize("case", SMALL)
def test_conv_small(case, layout, mode):
    say("conv", case, layout, mode)
    x, cache, wgt, b = inputs(case)
    got = run_gpu(x, cache, wgt, b, mode, layout)
    check(got, x, cache, wgt, b, mode, f"{case} {layout} {mode}")


@pytest.mark.parametrize("layout", ["ncthw", "nthwc"])
@pytest.mark.parametrize("case", HALO)
def test_conv_halo_tile_default(case, layout):
    say("conv", case, layout, "bf16")
    x, cache, wgt, b = inputs(case)
    got = run_gpu(x, cache, wgt, b, "bf16", layout)
    check(got, x, cache, wgt, b, "bf16", f"{case} {layout} bf16")


@pytest.fixture
def conv_kernel():
    try:
        yield wanvae.wanvae_set_conv_kernel
    finally:
        wanvae.wanvae_set_conv_kernel(-1)


@pytest.mark.parametrize("kernel", range(wanvae.CONV_KERNELS))
@pytest.mark.parametrize("case", SMALL + HALO[:1])
def test_conv_each_kernel_bf16(case, kernel, conv_kernel):
    """Every conv kernel, forced wherever it can run the conv, against the oracle."""
    say("conv", case, "kernel", kernel)
    conv_kernel(kernel)
    x, cache, wgt, b = inputs(case)
    got = run_gpu(x, cache, wgt, b, "bf16", "nthwc")
    check(got, x, cache, wgt, b, "bf16", f"{case} kernel {kernel}")



def test_conv_is_deterministic_and_zero_history_equals_no_history():
    g = np.random.default_rng(5)
    x = g.standard_normal((1, 64, 2, 6, 40)).astype(np.float32)
    w = (g.standard_normal((128, 64, 3, 3, 3)) / 40).astype(np.float32)
    b = np.zeros(128, np.float32)
    a1 = run_gpu(x, None, w, b, "bf16", "nthwc")
    a2 = run_gpu(x, None, w, b, "bf16", "nthwc")
    z = run_gpu(x, np.zeros((1, 64, 2, 6, 40), np.float32), w, b, "bf16", "nthwc")
    assert np.array_equal(a1, a2) and np.array_equal(a1, z)


def sample_points(shape, n, seed):
    g = np.random.default_rng(seed)
    B, Co, t, h, w = shape
    pts = np.stack([g.integers(0, s, n) for s in (B, Co, t, h, w)], 1)
    # the borders, where the padding matters
    edge = np.array([[0, c, tt, y, xx] for c in (0, Co - 1) for tt in (0, t - 1) for y in (0, h - 1) for xx in (0, w - 1)])
    return np.concatenate([pts, edge])


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("name", list(synthetic.CONV_CONFIGS))
def test_conv_full_size_sampled(name, mode):
    cfg = synthetic.CONV_CONFIGS[name]
    say("conv full", name, mode)
    x, cache, w, b = cfg.tensors()
    xt = to_dev(x, mode).permute(0, 2, 3, 4, 1).contiguous()
    ct = to_dev(cache, mode).permute(0, 2, 3, 4, 1).contiguous()
    y = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(w, mode), to_dev(b, mode), layout="nthwc")
    torch.cuda.synchronize()
    pts = sample_points((1, cfg.C, cfg.t, cfg.h, cfg.w), 3000, 77)
    got = y[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 4], pts[:, 1]].float().cpu().numpy()
    xs = np.concatenate([rounded(cache, mode), rounded(x, mode)], 2)
    want = oracle.conv_points(xs, rounded(w, mode), rounded(b, mode), pts)
    wr = rounded(w, mode)
    err = acc_bound(wr[0].size, oracle.conv_points(np.abs(xs), np.abs(wr), np.abs(rounded(b, mode)), pts))
    if mode == "bf16":
        assert_bf16_close(got, oracle.round_bf16(want), err, min_exact=0.97, what=name)
    else:
        d = np.abs(got - want)
        assert np.all(d <= err + 2.0 ** -24 * np.abs(want)), d.max()
        assert d.max() <= 1e-3, d.max()


# ------------------------------------------------------------------ float32 output, cache_out

def run_gpu_f32_out(x, cache, w, b, layout):
    """The bf16 conv with a float32 y, and the same conv's bf16 y."""
    xt, wt, bt = to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "bf16")
    ct = to_dev(cache, "bf16") if cache is not None and cache.shape[2] else None
    if layout == "nthwc":
        xt = xt.permute(0, 2, 3, 4, 1).contiguous()
        ct = ct.permute(0, 2, 3, 4, 1).contiguous() if ct is not None else None
    y32 = wanvae.wanvae_causal_conv3d(xt, ct, wt, bt, layout=layout, y_dtype=torch.float32)
    y16 = wanvae.wanvae_causal_conv3d(xt, ct, wt, bt, layout=layout)
    torch.cuda.synchronize()
    assert y32.dtype == torch.float32 and y16.dtype == torch.bfloat16
    y32, y16 = to_np(y32), to_np(y16)
    if layout == "nthwc":
        y32, y16 = y32.transpose(0, 4, 1, 2, 3), y16.transpose(0, 4, 1, 2, 3)
    return y32, y16


def check_f32_out(y32, y16, x, cache, w, b, what):
    """bf16 operands, float32 sums stored unrounded: within the float32 summation bound of the
    exact sum of the bf16-rounded operands; and rounding y32 to bf16 gives the bf16 output bit
    for bit (the same sums, one rounding later)."""
    xr, cr, wr, br = (rounded(a, "bf16") if a is not None else None for a in (x, cache, w, b))
    hist = cr if cr is not None and cr.shape[2] else None
    want = oracle.causal_conv(xr, wr, br, hist, oracle.Prec("fp64"))
    mag = oracle.causal_conv(np.abs(xr), np.abs(wr), np.abs(br), None if hist is None else np.abs(hist),
                             oracle.Prec("fp64"))
    err = acc_bound(w[0].size, mag) + 2.0 ** -24 * np.abs(want)
    d = np.abs(y32.astype(np.float64) - want)
    assert np.all(d <= err), f"{what}: max diff {d.max():.3g}, worst over bound {(d - err).max():.3g}"
    assert np.array_equal(oracle.round_bf16(y32), y16), what


@pytest.mark.parametrize("layout", ["ncthw", "nthwc"])
@pytest.mark.parametrize("case", SMALL + HALO)
def test_conv_bf16_float32_output(case, layout):
    say("conv f32 out", case, layout)
    x, cache, wgt, b = inputs(case)
    y32, y16 = run_gpu_f32_out(x, cache, wgt, b, layout)
    check_f32_out(y32, y16, x, cache, wgt, b, f"{case} {layout} y fp32")


@pytest.mark.parametrize("kernel", range(wanvae.CONV_KERNELS))
@pytest.mark.parametrize("case", SMALL[:2] + SMALL[5:] + HALO[:1])
def test_conv_float32_output_each_kernel(case, kernel, conv_kernel):
    """The float32-output epilogue of every conv kernel, forced wherever it can run the conv
    (the halo tiles, the direct-to-LDS tiles with and without split K, the register-staged
    tiles)."""
    say("conv f32 out", case, "kernel", kernel)
    conv_kernel(kernel)
    x, cache, wgt, b = inputs(case)
    y32, y16 = run_gpu_f32_out(x, cache, wgt, b, "nthwc")
    check_f32_out(y32, y16, x, cache, wgt, b, f"{case} kernel {kernel} y fp32")


@pytest.mark.parametrize("layout", ["ncthw", "nthwc"])
@pytest.mark.parametrize("mode", ["bf16", "fp32"])
@pytest.mark.parametrize("n_cache,t", [(0, 1), (0, 3), (1, 1), (1, 2), (2, 1), (2, 4)])
def test_conv_cache_out_is_the_last_frames(n_cache, t, mode, layout):
    """cache_out holds the last min(2, n_cache + t) frames of cache ++ x, bit for bit (the
    cache rule of the "Causal caches" section, as the oracle's cached conv keeps it), in the
    call's layout; y is unchanged by asking for it."""
    g = np.random.default_rng(100 + 10 * n_cache + t)
    B, C, h, w = 2, 40, 5, 7
    x = g.standard_normal((B, C, t, h, w)).astype(np.float32)
    cache = g.standard_normal((B, C, n_cache, h, w)).astype(np.float32)
    wgt = (g.standard_normal((24, C, 3, 3, 3)) / 20).astype(np.float32)
    b = np.zeros(24, np.float32)
    xt, ct = to_dev(x, mode), to_dev(cache, mode) if n_cache else None
    if layout == "nthwc":
        xt = xt.permute(0, 2, 3, 4, 1).contiguous()
        ct = ct.permute(0, 2, 3, 4, 1).contiguous() if ct is not None else None
    y, co = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(wgt, mode), to_dev(b, mode), layout=layout, return_cache=True)
    y0 = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(wgt, mode), to_dev(b, mode), layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    store = {}
    if n_cache:
        store["c"] = rounded(cache, mode)
    oracle.cached_conv(rounded(x, mode), rounded(wgt, mode), b, "c", store, oracle.Prec(mode))
    want = store["c"]
    got = to_np(co)
    if layout == "nthwc":
        got = got.transpose(0, 4, 1, 2, 3)
    assert got.shape == want.shape == (B, C, min(2, n_cache + t), h, w)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("layout", ["ncthw", "nthwc"])
def test_conv_cache_updated_in_place(layout):
    """cache_out may be the two-frame cache itself: after the call it holds the last two frames
    of cache ++ x, and y is the conv over the old cache."""
    g = np.random.default_rng(7)
    B, C, h, w = 1, 32, 6, 9
    x = g.standard_normal((B, C, 1, h, w)).astype(np.float32)
    cache = g.standard_normal((B, C, 2, h, w)).astype(np.float32)
    wgt = (g.standard_normal((32, C, 3, 3, 3)) / 20).astype(np.float32)
    b = np.zeros(32, np.float32)
    xt, ct = to_dev(x, "bf16"), to_dev(cache, "bf16")
    if layout == "nthwc":
        xt, ct = xt.permute(0, 2, 3, 4, 1).contiguous(), ct.permute(0, 2, 3, 4, 1).contiguous()
    y_ref = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(wgt, "bf16"), to_dev(b, "bf16"), layout=layout)
    y = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(wgt, "bf16"), to_dev(b, "bf16"), layout=layout, cache_out=ct)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    got = to_np(ct)
    if layout == "nthwc":
        got = got.transpose(0, 4, 1, 2, 3)
    want = np.concatenate([rounded(cache, "bf16")[:, :, 1:], rounded(x, "bf16")], 2)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", list(synthetic.CONV_CONFIGS))
def test_conv_full_size_float32_output_sampled(name):
    """The full-size convs with bf16 operands and a float32 y, at sampled outputs (each an
    oracle dot product), within the float32 summation bound; and the updated cache."""
    cfg = synthetic.CONV_CONFIGS[name]
    say("conv full f32 out", name)
    x, cache, w, b = cfg.tensors()
    xt = to_dev(x, "bf16").permute(0, 2, 3, 4, 1).contiguous()
    ct = to_dev(cache, "bf16").permute(0, 2, 3, 4, 1).contiguous()
    y, co = wanvae.wanvae_causal_conv3d(xt, ct, to_dev(w, "bf16"), to_dev(b, "bf16"), layout="nthwc",
                                        y_dtype=torch.float32, return_cache=True)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    pts = sample_points((1, cfg.C, cfg.t, cfg.h, cfg.w), 3000, 78)
    got = y[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 4], pts[:, 1]].cpu().numpy().astype(np.float64)
    xs = np.concatenate([rounded(cache, "bf16"), rounded(x, "bf16")], 2)
    wr, br = rounded(w, "bf16"), rounded(b, "bf16")
    want = oracle.conv_points(xs, wr, br, pts)
    err = acc_bound(wr[0].size, oracle.conv_points(np.abs(xs), np.abs(wr), np.abs(br), pts)) + 2.0 ** -24 * np.abs(want)
    d = np.abs(got - want)
    assert np.all(d <= err), (d.max(), (d - err).max())
    # the new cache: the last two frames of x (x has t >= 2 frames) or cache[1] ++ x
    want_c = xs[:, :, -2:].transpose(0, 2, 3, 4, 1)
    assert torch.equal(co.float().cpu(), torch.from_numpy(np.ascontiguousarray(want_c)))
