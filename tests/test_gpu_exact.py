"""The bf16 decode's rounding points, bit for bit (GPU).

With synthetic.exact_sum_weights every conv output is its bias plus at most one product, so
the GPU's float32 sums equal the oracle's float64 ones exactly, in any order. The only
differences left are those of the page's "Precision" section: where the decode rounds to
bf16. The RMS norm (whose float32 sum of squares still differs from the oracle's float64 one in
its last bits), the residual and DupUp3D sums, the time conv's interleave, the attention
block's residual, unpatchify and clamp are then checked bit for bit: at least 99.9% of the
video's values equal the oracle's, and every other one within 2^-7, one bf16 spacing at the top
of the video's range [-1, 1] (a norm whose float32 rounding lands on the other side of a bf16
rounding boundary moves one value by one spacing at that value's magnitude; a sum that
cancels to near zero keeps that absolute difference, so the bound is absolute). fp32 decodes
under the same weights agree with the oracle to float32 rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from _gpu import bf16_ulp, dev, say, to_np
from video_vae_decoding_amd import wanvae

pytestmark = pytest.mark.gpu

CASES = [
    # (base, B, T, h, w): the tiny decoder with two steady-state chunks (two frames of time-conv
    # history) and a ragged latent; base 32 on 8 x 12 latents (128-channel levels: the halo-tile
    # convs at levels 1-3, the level-0 split K); base 96 (the 4-wave 384-wide attention, and the
    # generic norm at 96 and 192 channels)
    (16, 2, 4, 3, 5),
    (32, 1, 3, 8, 12),
    (96, 1, 2, 2, 3),
]


def inputs(base, B, T, h, w):
    return synthetic.exact_sum_weights(base, 21), synthetic.normal(21, "latents", (B, synthetic.Z_DIM, T, h, w))


def gpu_decode(z, W, mode):
    Wt = {k: torch.from_numpy(v).to(dev()) for k, v in W.items()}
    got = wanvae.wanvae_decode(torch.from_numpy(z).to(dev()), Wt, torch.bfloat16 if mode == "bf16" else torch.float32)
    torch.cuda.synchronize()
    return got


def decode_both(base, B, T, h, w, mode):
    W, z = inputs(base, B, T, h, w)
    return to_np(gpu_decode(z, W, mode)).astype(np.float64), oracle.decode(z, W, mode).astype(np.float64)


@pytest.fixture
def norm_kernel():
    """Sets the norm kernel for one test and restores the default afterwards."""
    try:
        yield wanvae.wanvae_set_norm_kernel
    finally:
        wanvae.wanvae_set_norm_kernel(-1)


@pytest.mark.parametrize("silu", ["auto", "table"])
@pytest.mark.parametrize("case", CASES)
def test_exact_sum_decode_bf16_bit_level(case, silu, norm_kernel):
    """silu = "table": every bf16 norm reads its SiLU from the LDS table (by default only the
    large launches do, and these decoders have none)."""
    say("exact-sum bf16 decode", case, silu)
    norm_kernel(1 if silu == "table" else -1)
    got, want = decode_both(*case, "bf16")
    assert got.shape == want.shape
    d = np.abs(got - want)
    exact = float(np.mean(d == 0))
    ulp = bf16_ulp(np.maximum(np.abs(got), np.abs(want)))
    say(case, "bit-equal", exact, "max diff", d.max(), "max diff / spacing", (d / ulp).max())
    assert exact >= 0.999, exact
    assert d.max() <= 2.0 ** -7, d.max()


@pytest.mark.parametrize("case", CASES)
def test_silu_table_and_arithmetic_give_the_same_bits(case, norm_kernel):
    """The bf16 decode with every norm's SiLU from the LDS table equals, bit for bit, the decode
    with every SiLU computed."""
    say("SiLU table against arithmetic", case)
    W, z = inputs(*case)
    norm_kernel(1)
    tab = gpu_decode(z, W, "bf16")
    norm_kernel(0)
    ari = gpu_decode(z, W, "bf16")
    assert torch.equal(tab, ari)


@pytest.mark.parametrize("case", CASES[:2])
def test_exact_sum_decode_fp32(case):
    say("exact-sum fp32 decode", case)
    got, want = decode_both(*case, "fp32")
    d = np.abs(got - want)
    say(case, "max diff", d.max(), "bit-equal", float(np.mean(d == 0)))
    assert d.max() <= 1e-5, d.max()
