"""The C-ABI library on the CPU: it loads, exports every entry point include/wanvae.h
declares, and rejects bad arguments with the documented status before launching anything
(validation never dereferences the data pointers, so host pointers stand in for device ones)."""
import ctypes
import os
import re

import pytest
import torch

import synthetic
from video_vae_decoding_amd import wanvae as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "wanvae.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wanvae_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"wanvae_decode", "wanvae_causal_conv3d", "wanvae_attn_block", "wanvae_last_error"} <= set(names)
    L = W.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.wanvae_version() >= 200


def host_weights(base=16):
    # host tensors: only shapes, dtypes and pointers are read by the validation
    return {k: torch.zeros(s) for k, s in synthetic.weight_shapes(base).items()}


def ws_size(weights, dtype=W.F32, B=1, T=2, h=4, w=4):
    arr, n = W.tensor_table(weights)
    out = ctypes.c_size_t(0)
    rc = W.lib().wanvae_decode_workspace_size(B, T, h, w, arr, n, dtype, ctypes.byref(out))
    return rc, out.value


def test_workspace_size_grows_with_the_problem():
    wts = host_weights()
    rc, small = ws_size(wts)
    assert rc == W.OK and small > 0
    assert ws_size(wts, T=5)[1] > small
    assert ws_size(wts, B=2)[1] > small
    assert ws_size(wts, dtype=W.BF16)[1] < small


def full_table(base=256):
    """A parameter table with the full decoder's shapes and dummy pointers (nothing is read)."""
    items = list(synthetic.weight_shapes(base).items())
    tab = (W.wanvae_tensor * len(items))()
    for i, (k, s) in enumerate(items):
        tab[i] = W.wanvae_tensor(k.encode(), 4096, W.F32, len(s), (ctypes.c_int64 * 5)(*s, *([0] * (5 - len(s)))))
    return tab, len(items)


def test_decode_workspace_for_the_full_decoder_fits_one_gpu():
    tab, n = full_table()
    out = ctypes.c_size_t(0)
    assert W.lib().wanvae_decode_workspace_size(1, 31, 44, 80, tab, n, W.BF16, ctypes.byref(out)) == W.OK
    assert 5e9 < out.value < 40e9, out.value
    assert W.lib().wanvae_decode_workspace_size(2, 31, 44, 80, tab, n, W.F32, ctypes.byref(out)) == W.OK
    assert out.value < 150e9, out.value


def call_decode(weights, dtype=W.F32, z_dtype=W.F32, B=1, T=2, h=4, w=4, z=4096, video=4096, ws=4096, ws_bytes=1 << 40):
    arr, n = W.tensor_table(weights)
    return W.lib().wanvae_decode(z, z_dtype, B, T, h, w, arr, n, dtype, video, ws, ws_bytes, None)


def test_bad_dtype_is_edtype():
    assert call_decode(host_weights(), dtype=2) == W.EDTYPE
    assert "WANVAE_F32" in W.lib().wanvae_last_error().decode()
    assert call_decode(host_weights(), z_dtype=7) == W.EDTYPE
    with pytest.raises(ValueError):
        W.check(W.EDTYPE)


def test_missing_parameter_is_emissing():
    wts = host_weights()
    del wts["decoder.up_blocks.1.upsampler.time_conv.bias"]
    assert call_decode(wts) == W.EMISSING
    assert "time_conv.bias" in W.lib().wanvae_last_error().decode()


def test_wrong_shape_is_eshape():
    wts = host_weights()
    wts["decoder.mid_block.resnets.1.conv2.weight"] = torch.zeros(64, 64, 3, 3, 1)
    assert call_decode(wts) == W.ESHAPE
    wts = host_weights()
    wts["decoder.norm_out.gamma"] = torch.zeros(15)
    assert call_decode(wts) == W.ESHAPE
    assert call_decode(host_weights(), T=0) == W.ESHAPE


def test_gamma_of_any_shape_with_C_elements_is_accepted():
    wts = host_weights()
    wts["decoder.norm_out.gamma"] = torch.zeros(16)
    wts["decoder.mid_block.attentions.0.norm.gamma"] = torch.zeros(1, 64)
    assert ws_size(wts)[0] == W.OK


def test_other_topology_is_etopology():
    assert call_decode(host_weights(base=8)) == W.ETOPOLOGY
    # widths the mid-block attention does not run (4 * base = 192, 320, 448): rejected with the
    # other arguments, before any launch
    for base in (48, 80, 112):
        assert call_decode(host_weights(base=base)) == W.ETOPOLOGY, base
        assert "decoder_base_dim" in W.lib().wanvae_last_error().decode()
        assert ws_size(host_weights(base=base))[0] == W.ETOPOLOGY
    for base in (16, 32, 64, 96, 128):
        assert ws_size(host_weights(base=base))[0] == W.OK, base
    wts = host_weights()
    wts["post_quant_conv.weight"] = torch.zeros(16, 16, 1, 1, 1)
    assert call_decode(wts) == W.ETOPOLOGY


def test_duplicate_names_and_null_pointers_are_earg():
    wts = host_weights()
    arr, n = W.tensor_table(wts)
    dup = (W.wanvae_tensor * (n + 1))(*arr[:n], arr[0])
    assert W.lib().wanvae_decode(4096, 0, 1, 2, 4, 4, dup, n + 1, 0, 4096, 4096, 1 << 40, None) == W.EARG
    assert call_decode(wts, z=None) == W.EARG


def test_names_outside_the_prefixes_are_ignored():
    wts = host_weights()
    wts["encoder.conv_in.weight"] = torch.zeros(3)
    wts["encoder.conv_in.weight2"] = torch.zeros(3)
    assert ws_size(wts)[0] == W.OK


def test_small_workspace_is_eworkspace():
    wts = host_weights()
    _, need = ws_size(wts)
    assert call_decode(wts, ws_bytes=need - 1) == W.EWORKSPACE


def test_conv_and_attention_validation():
    L = W.lib()
    w = W.tensor_struct("weight", torch.zeros(16, 24, 3, 3, 3))
    b = W.tensor_struct("bias", torch.zeros(16))
    args = dict(x=4096, cache=4096, B=1, Cin=24, t=2, h=4, w=4, n=2)

    def conv(**kw):
        a = {**args, **kw}
        return L.wanvae_causal_conv3d(a["x"], a["cache"], a["B"], a["Cin"], a["t"], a["h"], a["w"], a["n"],
                                      ctypes.byref(w), ctypes.byref(b), kw.get("layout", 0), kw.get("dtype", 0),
                                      kw.get("y", 8192), kw.get("y_dtype", kw.get("dtype", 0)), kw.get("cache_out"),
                                      4096, 1 << 40, None)
    assert conv(dtype=3) == W.EDTYPE
    assert conv(dtype=W.BF16, y_dtype=5) == W.EDTYPE
    assert conv(dtype=W.F32, y_dtype=W.BF16) == W.EDTYPE   # a float32 conv returns float32
    assert "y_dtype" in L.wanvae_last_error().decode()
    assert conv(Cin=20) == W.ESHAPE        # not a multiple of 8 / does not match the weight
    assert conv(n=3) == W.ESHAPE
    assert conv(t=7) == W.ESHAPE
    assert conv(cache=None) == W.EARG
    assert conv(layout=5) == W.EARG
    assert conv(x=4096 + 8) == W.EARG      # 16-byte alignment
    assert conv(y=8192 + 4, y_dtype=W.F32) == W.EARG
    assert conv(cache_out=12288 + 2) == W.EARG
    assert conv(y=4096) == W.EARG          # y aliases x
    assert conv(cache_out=8192) == W.EARG  # cache_out aliases y
    assert conv(cache_out=4096) == W.EARG  # cache_out aliases x
    assert conv(n=1, cache_out=4096 + 16, cache=4096 + 16) == W.EARG  # in place needs two cache frames
    g = W.tensor_struct("gamma", torch.zeros(64))
    qw = W.tensor_struct("qkv_w", torch.zeros(192, 64, 1, 1))
    qb = W.tensor_struct("qkv_b", torch.zeros(192))
    pw = W.tensor_struct("proj_w", torch.zeros(64, 64, 1, 1))
    pb = W.tensor_struct("proj_b", torch.zeros(64))

    def attn(C=64, x=4096, y=8192, dtype=0, gam=g):
        return L.wanvae_attn_block(x, 0, 1, C, 2, 3, 3, ctypes.byref(gam), ctypes.byref(qw), ctypes.byref(qb),
                                   ctypes.byref(pw), ctypes.byref(pb), dtype, y, 4096, 1 << 40, None)
    assert attn(dtype=9) == W.EDTYPE
    assert attn(C=96) == W.ESHAPE
    assert attn(C=192) == W.ESHAPE         # a multiple of 64 the attention kernels do not run
    assert "384" in L.wanvae_last_error().decode()
    assert attn(y=4096) == W.EARG
    assert attn(gam=W.tensor_struct("gamma", torch.zeros(63))) == W.ESHAPE


def test_conv_kernel_selection_range():
    try:
        for k in range(-1, W.CONV_KERNELS):
            W.wanvae_set_conv_kernel(k)
        for bad in (-2, W.CONV_KERNELS):
            with pytest.raises(ValueError):
                W.wanvae_set_conv_kernel(bad)
    finally:
        W.wanvae_set_conv_kernel(-1)


def test_decode_pipeline_switch():
    L = W.lib()
    try:
        assert L.wanvae_set_decode_pipeline(0) == W.OK
        assert L.wanvae_set_decode_pipeline(1) == W.OK
        for bad in (-1, 2):
            assert L.wanvae_set_decode_pipeline(bad) == W.EARG
            assert "0 or 1" in L.wanvae_last_error().decode()
    finally:
        W.wanvae_set_decode_pipeline(True)


def test_norm_kernel_switch():
    L = W.lib()
    try:
        for mode in (-1, 0, 1):
            assert L.wanvae_set_norm_kernel(mode) == W.OK
        for bad in (-2, 2):
            assert L.wanvae_set_norm_kernel(bad) == W.EARG
            assert "-1, 0 or 1" in L.wanvae_last_error().decode()
            with pytest.raises(ValueError):
                W.wanvae_set_norm_kernel(bad)
    finally:
        W.wanvae_set_norm_kernel(-1)


def tiled_ws(tab, n, dtype=W.BF16, B=1, T=31, h=44, w=80, tile=(256, 256), stride=(192, 192)):
    out = ctypes.c_size_t(0)
    rc = W.lib().wanvae_decode_tiled_workspace_size(B, T, h, w, tab, n, dtype, tile[0], tile[1], stride[0], stride[1],
                                                    ctypes.byref(out))
    return rc, out.value


def test_tiled_decode_validation_and_workspace():
    """The tiled decode's arguments are checked before anything runs, and at the page's default
    tile (256, stride 192) its workspace for the 704 x 1280 x 121 decode is a fraction of the
    untiled decode's (the point of tiling)."""
    tab, n = full_table()
    rc, tiled = tiled_ws(tab, n)
    assert rc == W.OK
    out = ctypes.c_size_t(0)
    assert W.lib().wanvae_decode_workspace_size(1, 31, 44, 80, tab, n, W.BF16, ctypes.byref(out)) == W.OK
    assert tiled < 0.6 * out.value, (tiled, out.value)
    for tile, stride in (((250, 256), (192, 192)), ((256, 256), (0, 192)), ((256, 256), (272, 192)),
                         ((256, 256), (192, 200))):
        assert tiled_ws(tab, n, tile=tile, stride=stride)[0] == W.EARG
    assert tiled_ws(tab, n, dtype=7)[0] == W.EDTYPE
    # one tile covering the video: the untiled decode's buffers plus the tile rows
    assert tiled_ws(tab, n, h=4, w=4, T=2, tile=(64, 64), stride=(64, 64))[0] == W.OK
    wts = host_weights()
    arr, m = W.tensor_table(wts)
    _, need = tiled_ws(arr, m, dtype=W.F32, T=2, h=4, w=4, tile=(32, 32), stride=(16, 16))
    assert W.lib().wanvae_decode_tiled(4096, W.F32, 1, 2, 4, 4, arr, m, W.F32, 32, 32, 16, 16, 4096, 4096, need - 1,
                                       None) == W.EWORKSPACE
    assert W.lib().wanvae_decode_tiled(None, W.F32, 1, 2, 4, 4, arr, m, W.F32, 32, 32, 16, 16, 4096, 4096, need,
                                       None) == W.EARG


def test_oversized_latent_is_eshape_before_any_launch():
    """A latent past the library's size limit (B * h * w * 4096 above 2^31: the kernels use
    32-bit offsets inside a frame) is rejected before anything runs, as are zero sizes."""
    wts = host_weights()
    assert call_decode(wts, h=1000, w=1000) == W.ESHAPE
    assert "too large" in W.lib().wanvae_last_error().decode()
    assert call_decode(wts, B=0) == W.ESHAPE
    assert call_decode(wts, w=0) == W.ESHAPE
    tab, n = full_table()
    assert tiled_ws(tab, n, h=1000, w=1000)[0] == W.ESHAPE
