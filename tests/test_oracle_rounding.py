"""Pins of the oracle's bf16 rounding points outside the convs (CPU only).

FastVideo's "wan22_vae_decode reference.py" page, section "Precision", lists where a bf16
decode rounds: the weights and the latents are cast to bf16 first; every conv returns bf16;
the RMS norm rounds after normalising and after each product; SiLU, the residual sums,
DupUp3D and unpatchify run in bf16 tensors, so each sum is rounded. In float64 every one of
these roundings is the identity, so only bf16-specific pins catch a dropped one. Each test
below fails if one rounding point is removed from the oracle:

* the latents and weights: a bf16 decode depends on them only through their bf16 values;
* the residual sum and the up block's DupUp3D sum: closed forms whose exact sum lies 3/4 of a
  bf16 spacing above 1, so the rounded and the unrounded sums differ;
* the residual block as a whole: re-evaluated with torch's own bf16 tensor arithmetic.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic
from oracle.decoder import residual_block, up_block

PBF = oracle.Prec("bf16")
P64 = oracle.Prec("fp64")

B_SMALL = 3 * 2.0 ** -9            # exactly representable in bf16 (binary 1.1 x 2^-8)
ONE_PLUS_B_BF16 = 1.0078125         # bf16(1 + 3*2^-9): 1 + 3/4 of the spacing 2^-7 rounds up


def _is_bf16(a):
    a = np.asarray(a, np.float32)
    return np.array_equal(oracle.round_bf16(a), a)


def test_closed_form_constants():
    assert _is_bf16([B_SMALL, 1.0, ONE_PLUS_B_BF16])
    assert float(torch.tensor(1.0 + B_SMALL, dtype=torch.float32).to(torch.bfloat16)) == ONE_PLUS_B_BF16
    assert 1.0 + B_SMALL != ONE_PLUS_B_BF16


def test_bf16_decode_depends_on_weights_and_latents_only_through_their_bf16_values():
    """'Precision': the latents and every weight are cast to bf16 before anything runs. So
    decoding the float32 inputs must equal decoding their bf16 roundings, bit for bit, while the
    roundings do change the inputs (and a decode of unrounded values would differ)."""
    z = synthetic.normal(11, "latents", (1, synthetic.Z_DIM, 2, 3, 3))
    W = synthetic.gen_weights(16, 11, 0.1)
    assert not _is_bf16(z)
    assert all(not _is_bf16(v) for k, v in W.items() if k.endswith(".weight"))
    got = oracle.decode(z, W, "bf16")
    zr = oracle.round_bf16(z)
    Wr = {k: oracle.round_bf16(v) for k, v in W.items()}
    assert np.array_equal(oracle.decode(zr, Wr, "bf16"), got)
    # each of the two roundings matters on its own: with only one of them applied the
    # (unrounded) other input changes the bf16 video
    assert not np.array_equal(oracle.decode(zr, W, "fp32"), oracle.decode(zr, Wr, "fp32"))
    assert not np.array_equal(oracle.decode(z, Wr, "fp32"), oracle.decode(zr, Wr, "fp32"))


def test_fp32_decode_depends_on_inputs_only_through_their_fp32_values():
    g = np.random.default_rng(12)
    z = g.standard_normal((1, synthetic.Z_DIM, 2, 2, 3))
    W = {k: v.astype(np.float64) * (1 + 1e-9 * g.standard_normal(v.shape))
         for k, v in synthetic.gen_weights(16, 12, 0.1).items()}
    got = oracle.decode(z, W, "fp32")
    W32 = {k: v.astype(np.float32) for k, v in W.items()}
    assert np.array_equal(oracle.decode(z.astype(np.float32), W32, "fp32"), got)


def _bf16_weights(base):
    W = synthetic.gen_weights(base, 13, 0.1)
    return {k: oracle.round_bf16(v) for k, v in W.items()}


@pytest.mark.parametrize("name,C", [("decoder.mid_block.resnets.0", 64), ("decoder.up_blocks.2.resnets.0", 64)])
def test_residual_sum_is_rounded_closed_form(name, C):
    """conv2 weights zero and bias 3*2^-9 make conv2's output that bias; with x = 1 the block's
    sum is 1 + 3*2^-9, which bf16 holds only as 1.0078125 ('Precision': the sums run in bf16).
    Up block 2's first resnet has a 1x1 shortcut (64 -> 32): its weights zero and bias 1 make
    the shortcut 1 as well. fp64 keeps the exact sum."""
    W = _bf16_weights(16)
    co = W[f"{name}.conv2.weight"].shape[0]
    W[f"{name}.conv2.weight"] = np.zeros_like(W[f"{name}.conv2.weight"])
    W[f"{name}.conv2.bias"] = np.full(co, B_SMALL, np.float32)
    if f"{name}.conv_shortcut.weight" in W:
        W[f"{name}.conv_shortcut.weight"] = np.zeros_like(W[f"{name}.conv_shortcut.weight"])
        W[f"{name}.conv_shortcut.bias"] = np.ones(co, np.float32)
    x = np.ones((1, C, 2, 3, 4), np.float32)
    out = residual_block(x, W, name, {}, PBF)
    assert out.shape == (1, co, 2, 3, 4)
    assert np.all(out == np.float32(ONE_PLUS_B_BF16))
    out64 = residual_block(x.astype(np.float64), W, name, {}, P64)
    assert np.all(out64 == 1.0 + B_SMALL)


@pytest.mark.parametrize("u,first", [(0, True), (0, False), (1, False), (2, True), (2, False)])
def test_dup_up_sum_is_rounded_closed_form(u, first):
    """The up block adds DupUp3D of its input to the upsampler's output. With the upsampling
    conv's weights zero and its bias 3*2^-9, and the block input 1 everywhere (DupUp3D copies
    it), the block's output is bf16(1 + 3*2^-9) = 1.0078125 at every position, whatever the
    residual blocks and the time conv compute ('Precision': DupUp3D and the sums run in bf16)."""
    base = 16
    W = _bf16_weights(base)
    name = f"decoder.up_blocks.{u}.upsampler.resample.1"
    co = W[f"{name}.weight"].shape[0]
    W[f"{name}.weight"] = np.zeros_like(W[f"{name}.weight"])
    W[f"{name}.bias"] = np.full(co, B_SMALL, np.float32)
    ci = synthetic.up_blocks(base)[u][0]
    temporal = synthetic.up_blocks(base)[u][2]
    x = np.ones((1, ci, 1, 2, 3), np.float32)
    out = up_block(x, W, u, {}, first, PBF)
    ft = 2 if (temporal and not first) else 1
    assert out.shape == (1, co, ft, 4, 6)
    assert np.all(out == np.float32(ONE_PLUS_B_BF16))
    out64 = up_block(x.astype(np.float64), W, u, {}, first, P64)
    assert np.all(out64 == 1.0 + B_SMALL)


def _torch_bf16_residual_block(x, W, name):
    """The residual block in torch's CPU bf16 tensor arithmetic: F.normalize on the float32
    values then a bf16 tensor; the products by sqrt(C) and gamma, SiLU and the final sum on
    bf16 tensors (torch rounds each result to bf16); each causal conv as F.conv3d in float64 on
    the bf16 values with two zero frames in front, rounded once to bf16 (fp32-accumulating
    kernels give this up to ties)."""
    bf = torch.bfloat16

    def norm_silu(h, g):
        C = h.shape[1]
        hn = F.normalize(h.float(), dim=1).to(bf)
        y = hn * C ** 0.5 * torch.from_numpy(g).to(bf)
        return F.silu(y)

    def conv(h, w, b):
        hp = F.pad(h.double(), (1, 1, 1, 1, 2, 0))
        return F.conv3d(hp, torch.from_numpy(w).double(), torch.from_numpy(b).double()).to(bf)

    xt = torch.from_numpy(x).to(bf)
    h = conv(norm_silu(xt, W[f"{name}.norm1.gamma"]), W[f"{name}.conv1.weight"], W[f"{name}.conv1.bias"])
    h = conv(norm_silu(h, W[f"{name}.norm2.gamma"]), W[f"{name}.conv2.weight"], W[f"{name}.conv2.bias"])
    return (h + xt).float().numpy()


def test_residual_block_matches_torch_bf16_arithmetic():
    name = "decoder.mid_block.resnets.0"
    W = _bf16_weights(16)
    x = oracle.round_bf16(synthetic.normal(14, "x", (1, 64, 3, 4, 5)))
    got = residual_block(x, W, name, {}, PBF)
    want = _torch_bf16_residual_block(x, W, name)
    # ties and float64 vs float32 norms may round apart by one spacing, which the second
    # conv can carry; most values agree bit for bit
    d = np.abs(got.astype(np.float64) - want)
    assert np.mean(d == 0) > 0.97, np.mean(d == 0)
    assert np.all(d <= 4 * 2.0 ** -7 * np.maximum(np.abs(want), 1.0)), d.max()
    # the unrounded sum would not be a bf16 value in most positions
    unrounded = residual_block(x, W, name, {}, oracle.Prec("fp32"))
    assert np.mean(unrounded == want) < 0.5


@pytest.mark.parametrize("base,h,w,T", [(16, 3, 5, 4), (32, 4, 6, 2)])
def test_exact_sum_weights_make_the_decode_independent_of_the_summation_order(base, h, w, T):
    """Under synthetic.exact_sum_weights every conv output is its bias plus at most one product
    (each a bf16 times a power of two), so its float32 sum is exact in any order: the oracle's
    bf16 decode with float64 sums and with float32 sums agree bit for bit. What remains are the
    rounding points themselves, which move the video well away from the fp32 decode. This is
    the construction the GPU's bit-level bf16 decode test relies on."""
    W = synthetic.exact_sum_weights(base, 3)
    z = synthetic.normal(3, "latents", (1, synthetic.Z_DIM, T, h, w))
    a = oracle.decode(z, W, "bf16")
    assert np.array_equal(a, oracle.decode(z, W, "bf16", acc="f32"))
    f = oracle.decode(z, W, "fp32")
    assert np.mean(np.abs(a.astype(np.float64) - f)) > 1e-4
    for k, v in W.items():
        assert _is_bf16(v), k
        if k.endswith(".weight"):
            nz = (v.reshape(v.shape[0], -1) != 0).sum(axis=1)
            assert np.all(nz == (0 if k.endswith("attentions.0.proj.weight") else 1)), k
