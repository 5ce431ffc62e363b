"""The allocation-free single conv (wanvae_causal_conv3d_noalloc) against wanvae_causal_conv3d.

Both run the same kernels on the same arguments, the first on the library's fixed device
scratch, the second on a workspace it is given: the outputs must agree bit for bit. Two calls
in a row on the scratch, the second smaller (the scratch keeps the first call's contents), then
a conv whose workspace exceeds the scratch, refused before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

from video_vae_decoding_amd import wanvae as W


def _conv_inputs(seed, B, C, Co, t, h, w, n_cache, layout, dev):
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal((B, C, t, h, w)).astype(np.float32))
    c = torch.from_numpy(g.standard_normal((B, C, n_cache, h, w)).astype(np.float32)) if n_cache else None
    wt = torch.from_numpy((g.standard_normal((Co, C, 3, 3, 3)) / np.sqrt(27 * C)).astype(np.float32))
    bt = torch.from_numpy((0.1 * g.standard_normal(Co)).astype(np.float32))
    x = x.to(dev).to(torch.bfloat16)
    c = c.to(dev).to(torch.bfloat16) if c is not None else None
    if layout == "nthwc":
        x = x.permute(0, 2, 3, 4, 1).contiguous()
        c = c.permute(0, 2, 3, 4, 1).contiguous() if c is not None else None
    return x, c, wt.to(dev), bt.to(dev)


@pytest.mark.gpu
def test_noalloc_conv_matches_the_workspace_conv_twice():
    dev = torch.device("cuda:0")
    cases = [
        # the 1024-channel level-0 conv with two cached frames (split K: the partial sums live in
        # the scratch), channels last, bf16 y
        dict(seed=1, B=1, C=1024, Co=1024, t=1, h=44, w=80, n_cache=2, layout="nthwc", y_dtype=torch.bfloat16),
        # then a smaller one, channels first (converted copies in the scratch), float32 y, cache_out
        dict(seed=2, B=2, C=64, Co=128, t=2, h=20, w=36, n_cache=1, layout="ncthw", y_dtype=torch.float32),
    ]
    for cs in cases:
        print("noalloc conv", cs, flush=True)
        x, c, wt, bt = _conv_inputs(cs["seed"], cs["B"], cs["C"], cs["Co"], cs["t"], cs["h"], cs["w"], cs["n_cache"],
                                    cs["layout"], dev)
        want, want_c = W.wanvae_causal_conv3d(x, c, wt, bt, layout=cs["layout"], y_dtype=cs["y_dtype"],
                                              return_cache=True)
        y = torch.empty_like(want)
        co = torch.empty_like(want_c)
        got = W.wanvae_causal_conv3d_noalloc(x, c, wt, bt, y, layout=cs["layout"], cache_out=co)
        torch.cuda.synchronize()
        assert got.data_ptr() == y.data_ptr()
        assert torch.equal(got, want), (got.float() - want.float()).abs().max()
        assert torch.equal(co, want_c)


def test_noalloc_conv_larger_than_the_scratch_is_eworkspace():
    """Validated and sized on the host: a conv needing more than the 128 MiB scratch (here
    2,048 channels: 226 MB of repacked weights) is refused before any launch or device call."""
    L = W.lib()
    # descriptors only: validation and sizing read no data
    w = W.wanvae_tensor(b"weight", 4096, W.BF16, 5, (ctypes.c_int64 * 5)(2048, 2048, 3, 3, 3))
    b = W.wanvae_tensor(b"bias", 4096, W.F32, 1, (ctypes.c_int64 * 5)(2048, 0, 0, 0, 0))
    rc = L.wanvae_causal_conv3d_noalloc(4096, None, 1, 2048, 1, 4, 4, 0, ctypes.byref(w), ctypes.byref(b), W.NTHWC,
                                        W.BF16, 8192, W.BF16, None, None)
    assert rc == W.EWORKSPACE
    assert "scratch" in L.wanvae_last_error().decode()
    # an invalid argument is still the argument error
    assert L.wanvae_causal_conv3d_noalloc(4096, None, 1, 2048, 1, 4, 4, 0, ctypes.byref(w), ctypes.byref(b), 7,
                                          W.BF16, 8192, W.BF16, None, None) == W.EARG
