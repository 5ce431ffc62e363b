"""Pins of the oracle's whole decoder (CPU only), on the tiny topology (decoder_base_dim 16).

The decoder has no worked example on the pages; its composition is pinned by the
invariants FastVideo's "wan22_vae_decode reference.py" page states: the frame count
4T - 3, causality (a chunk sees earlier ones only through the caches), independence of
the videos in a batch, and equality with the whole-sequence form of the section
"Causal caches".
"""
import numpy as np
import pytest

import oracle
import synthetic
from oracle.decoder import clamp, causal_conv, dup_up, rms_norm, silu, spatial_upsample, unpatchify, attention


def tiny(T=3, h=4, w=4, B=1, seed=0):
    z = synthetic.normal(seed, "latents", (B, synthetic.Z_DIM, T, h, w))
    return z, synthetic.gen_weights(16, seed, 0.1)


@pytest.mark.parametrize("T", [1, 2, 3])
def test_frame_count_is_4T_minus_3(T):
    z, W = tiny(T, 2, 3)
    v = oracle.decode(z, W, "fp32")
    assert v.shape == (1, 3, 4 * T - 3, 32, 48)
    assert np.all(np.abs(v) <= 1)


@pytest.mark.parametrize("mode", ["fp64", "bf16"])
def test_causal_prefix(mode):
    """Chunk i sees the earlier chunks only through the caches, so the first 4k - 3 frames of
    a decode are the decode of the first k latent frames, bit for bit."""
    z, W = tiny(4, 3, 3)
    full = oracle.decode(z, W, mode)
    for k in (1, 2, 3):
        assert np.array_equal(oracle.decode(z[:, :, :k], W, mode), full[:, :, :4 * k - 3])


def test_batch_independence():
    z, W = tiny(3, 3, 4, B=2)
    both = oracle.decode(z, W, "fp64")
    for b in range(2):
        np.testing.assert_allclose(oracle.decode(z[b:b + 1], W, "fp64"), both[b:b + 1], rtol=0, atol=1e-12)


def _whole_sequence_decode(z, Wt, P):
    """The whole-sequence form ('Causal caches', last paragraph): every causal conv over all
    frames of its level with two zero frames before the first; upsample3d's time conv over
    the frames after the first only, the first passing through; DupUp3D doubling every
    frame but the first. Built here from the oracle's pinned parts, without caches."""
    Wt = {k: P.R(v) for k, v in Wt.items()}

    def conv(x, name, kind="weight"):
        return causal_conv(x, Wt[f"{name}.weight"], Wt[f"{name}.bias"], None, P)

    def res(x, name):
        s = conv(x, f"{name}.conv_shortcut") if f"{name}.conv_shortcut.weight" in Wt else x
        h = conv(silu(rms_norm(x, Wt[f"{name}.norm1.gamma"], P), P), f"{name}.conv1")
        h = conv(silu(rms_norm(h, Wt[f"{name}.norm2.gamma"], P), P), f"{name}.conv2")
        return P.R(h.astype(np.float64) + s)

    x = conv(P.R(z), "post_quant_conv")
    x = conv(x, "decoder.conv_in")
    x = res(x, "decoder.mid_block.resnets.0")
    a = "decoder.mid_block.attentions.0"
    x = attention(x, Wt[f"{a}.norm.gamma"], Wt[f"{a}.to_qkv.weight"], Wt[f"{a}.to_qkv.bias"], Wt[f"{a}.proj.weight"], Wt[f"{a}.proj.bias"], P)
    x = res(x, "decoder.mid_block.resnets.1")
    for i, (ci, co, temporal, spatial) in enumerate(synthetic.up_blocks(16)):
        inp = x
        for j in range(3):
            x = res(x, f"decoder.up_blocks.{i}.resnets.{j}")
        if not spatial:
            continue
        if temporal and x.shape[2] > 1:
            y = conv(x[:, :, 1:], f"decoder.up_blocks.{i}.upsampler.time_conv")
            C = x.shape[1]
            inter = np.stack([y[:, :C], y[:, C:]], axis=3).reshape(y.shape[0], C, 2 * y.shape[2], *y.shape[3:])
            x = np.concatenate([x[:, :, :1], inter], axis=2)
        x = spatial_upsample(x, Wt[f"decoder.up_blocks.{i}.upsampler.resample.1.weight"], Wt[f"decoder.up_blocks.{i}.upsampler.resample.1.bias"], P)
        d = dup_up(inp, co, 2 if temporal else 1, first=False)
        if temporal:
            d = d[:, :, 1:]           # frame 0 keeps its last time copy only
        x = P.R(x.astype(np.float64) + d)
    x = silu(rms_norm(x, Wt["decoder.norm_out.gamma"], P), P)
    return clamp(unpatchify(conv(x, "decoder.conv_out")))


def test_chunk_loop_equals_whole_sequence_form():
    """Equal up to rounding (the page measured 1.7e-5 in fp32 with other conv shapes); in
    float64 the two orders of summation agree to 1e-10."""
    z, W = tiny(4, 3, 4)
    P = oracle.Prec("fp64")
    chunked = oracle.decode(z, W, "fp64")
    whole = _whole_sequence_decode(z, W, P)
    assert chunked.shape == whole.shape == (1, 3, 13, 48, 64)
    np.testing.assert_allclose(chunked, whole, rtol=0, atol=1e-10)
    # the video is not trivially clamped: most values lie inside (-1, 1)
    assert np.mean(np.abs(chunked) < 1) > 0.5


def test_names_outside_prefixes_are_ignored_and_missing_names_raise():
    z, W = tiny(1, 2, 2)
    ref = oracle.decode(z, W, "fp32")
    extra = dict(W)
    extra["encoder.conv_in.weight"] = np.full((3, 3), np.nan, np.float32)
    extra["quant_conv.weight"] = np.full((3, 3), np.nan, np.float32)
    assert np.array_equal(oracle.decode(z, extra, "fp32"), ref)
    missing = dict(W)
    del missing["decoder.up_blocks.2.upsampler.resample.1.bias"]
    with pytest.raises(KeyError):
        oracle.decode(z, missing, "fp32")


def test_rejects_other_dtypes():
    z, W = tiny(1, 2, 2)
    with pytest.raises(ValueError):
        oracle.decode(z, W, "fp16")


def test_bf16_decode_stays_close_to_fp32_decode():
    """The page reports its bf16 decode max 0.07, mean 0.003 from its fp32 decode (trained
    weights). Random init: the two modes stay within the same order."""
    z, W = tiny(2, 4, 4)
    a = oracle.decode(z, W, "fp32")
    b = oracle.decode(z, W, "bf16")
    d = np.abs(a - b)
    assert d.max() < 0.2 and d.mean() < 0.02
    assert oracle.psnr(a, b) > 30
