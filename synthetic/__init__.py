"""Seeded synthetic inputs for the Wan2.2 TI2V-5B VAE decoder.

This module is shared by the CPU oracle and the HIP path's tests and bench. It
holds no arithmetic of the method: only the parameter names and shapes of the
decoder (FastVideo's "wan22_vae_decode reference.py" page, module docstring
"What is computed" and the UP_BLOCKS / PREFIXES constants) and counter-free
numpy random streams.

Every tensor gets its own stream, ``default_rng([seed, crc32(name)])``, so no
value depends on the order in which tensors are drawn. Draws are float64
standard normals, scaled, then cast to float32. Shapes follow diffusers'
state-dict layout: conv3d weights [Co, Ci, kt, kh, kw], conv2d weights
[Co, Ci, kh, kw], biases [Co]. RMS-norm gammas are [C, 1, 1, 1] for the 3-D
norms and [C, 1, 1] for the attention norm, the shapes that broadcast over
[B, C, T, H, W] and [B*T, C, H, W] as the page's rms_norm multiplies them.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

Z_DIM = 48
PATCH = 2


def up_blocks(base: int):
    """(in channels, out channels, temporal upsample, spatial upsample) per up block."""
    c4, c2 = 4 * base, 2 * base
    return ((c4, c4, True, True), (c4, c4, True, True), (c4, c2, False, True), (c2, base, False, False))


def weight_shapes(base: int = 256, z_dim: int = Z_DIM) -> dict[str, tuple[int, ...]]:
    """The decoder's parameter table (110 tensors) for decoder_base_dim ``base``."""
    c = 4 * base
    s: dict[str, tuple[int, ...]] = {}
    s["post_quant_conv.weight"] = (z_dim, z_dim, 1, 1, 1)
    s["post_quant_conv.bias"] = (z_dim,)
    s["decoder.conv_in.weight"] = (c, z_dim, 3, 3, 3)
    s["decoder.conv_in.bias"] = (c,)

    def resnet(prefix, ci, co):
        s[f"{prefix}.norm1.gamma"] = (ci, 1, 1, 1)
        s[f"{prefix}.conv1.weight"] = (co, ci, 3, 3, 3)
        s[f"{prefix}.conv1.bias"] = (co,)
        s[f"{prefix}.norm2.gamma"] = (co, 1, 1, 1)
        s[f"{prefix}.conv2.weight"] = (co, co, 3, 3, 3)
        s[f"{prefix}.conv2.bias"] = (co,)
        if ci != co:
            s[f"{prefix}.conv_shortcut.weight"] = (co, ci, 1, 1, 1)
            s[f"{prefix}.conv_shortcut.bias"] = (co,)

    resnet("decoder.mid_block.resnets.0", c, c)
    a = "decoder.mid_block.attentions.0"
    s[f"{a}.norm.gamma"] = (c, 1, 1)
    s[f"{a}.to_qkv.weight"] = (3 * c, c, 1, 1)
    s[f"{a}.to_qkv.bias"] = (3 * c,)
    s[f"{a}.proj.weight"] = (c, c, 1, 1)
    s[f"{a}.proj.bias"] = (c,)
    resnet("decoder.mid_block.resnets.1", c, c)
    for i, (ci, co, temporal, spatial) in enumerate(up_blocks(base)):
        for j in range(3):
            resnet(f"decoder.up_blocks.{i}.resnets.{j}", ci if j == 0 else co, co)
        if temporal:
            s[f"decoder.up_blocks.{i}.upsampler.time_conv.weight"] = (2 * co, co, 3, 1, 1)
            s[f"decoder.up_blocks.{i}.upsampler.time_conv.bias"] = (2 * co,)
        if spatial:
            s[f"decoder.up_blocks.{i}.upsampler.resample.1.weight"] = (co, co, 3, 3)
            s[f"decoder.up_blocks.{i}.upsampler.resample.1.bias"] = (co,)
    s["decoder.norm_out.gamma"] = (base, 1, 1, 1)
    s["decoder.conv_out.weight"] = (3 * PATCH * PATCH, base, 3, 3, 3)
    s["decoder.conv_out.bias"] = (3 * PATCH * PATCH,)
    return s


def stream(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, zlib.crc32(name.encode())])


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws from the stream (seed, name)."""
    g = stream(seed, name)
    return (g.standard_normal(size=shape, dtype=np.float64) * std + mean).astype(np.float32)


def fan_in(shape) -> int:
    return int(np.prod(shape[1:]))


def gen_weights(base: int, seed: int, bias_std: float | None = None) -> dict[str, np.ndarray]:
    """Random-init weights: conv weights ~ N(0, 1/fan_in); biases ~ N(0, bias_std^2),
    or N(0, 1/fan_in of their conv) when bias_std is None; gammas 1 + 0.1 N(0, 1)."""
    shapes = weight_shapes(base)
    out = {}
    for name, shape in shapes.items():
        if name.endswith(".gamma"):
            out[name] = normal(seed, name, shape, 0.1, 1.0)
        elif name.endswith(".weight"):
            out[name] = normal(seed, name, shape, 1.0 / np.sqrt(fan_in(shape)))
        else:
            w = shapes[name[: -len("bias")] + "weight"]
            std = bias_std if bias_std is not None else 1.0 / np.sqrt(fan_in(w))
            out[name] = normal(seed, name, shape, std)
    return out


def exact_sum_weights(base: int, seed: int) -> dict[str, np.ndarray]:
    """Weights under which every conv output is its bias plus at most one product, so a
    float32 accumulation gives the exact sum in any order: each output channel of a conv has
    a single nonzero tap (a random input channel and tap) of value +-1 or +-1/2 (+-1/4 or
    +-1/2 for conv_out); the attention's output projection is zero. Biases are multiples of
    2^-8 in (-1/4, 1/4), gammas 1 + k/128 with |k| <= 16: every value is exact in bfloat16."""
    shapes = weight_shapes(base)
    out = {}
    for name, shape in shapes.items():
        g = stream(seed, name)
        if name.endswith(".gamma"):
            out[name] = (1.0 + g.integers(-16, 17, size=shape) / 128.0).astype(np.float32)
        elif name.endswith(".bias"):
            out[name] = (g.integers(-63, 64, size=shape) / 256.0).astype(np.float32)
        else:
            w = np.zeros(shape, np.float32)
            if not name.endswith("attentions.0.proj.weight"):
                co, ci = shape[0], shape[1]
                taps = int(np.prod(shape[2:]))
                flat = w.reshape(co, ci, taps)
                small = name == "decoder.conv_out.weight"
                mag = np.where(g.integers(0, 2, size=co) == 0, 0.5, 0.25 if small else 1.0)
                sign = np.where(g.integers(0, 2, size=co) == 0, 1.0, -1.0)
                flat[np.arange(co), g.integers(0, ci, size=co), g.integers(0, taps, size=co)] = mag * sign
            out[name] = w
    return out


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    base: int
    B: int
    T: int
    h: int
    w: int
    seed: int
    bias_std: float | None

    @property
    def frames(self) -> int:
        return 4 * self.T - 3

    def latents(self) -> np.ndarray:
        return normal(self.seed, "latents" if self.B == 1 else f"latents_b{self.B}", (self.B, Z_DIM, self.T, self.h, self.w))

    def weights(self) -> dict[str, np.ndarray]:
        return gen_weights(self.base, self.seed, self.bias_std)


# The decode workloads. tiny: decoder_base_dim 16, 2 latent frames of 4x4. small32:
# decoder_base_dim 32 (128-channel levels, the width the 3x3 halo-tile conv kernel needs),
# 2 latent frames of 8x12 (5 video frames of 128x192).
# ti2v5b_*: decoder_base_dim 256 at 704x1280 (landscape) or 1280x704 (portrait), 31 latent frames.
DECODE_CONFIGS = {
    "tiny": DecodeConfig("tiny", 16, 1, 2, 4, 4, 0, 0.1),
    "small32": DecodeConfig("small32", 32, 1, 2, 8, 12, 5, 0.1),
    "ti2v5b_landscape": DecodeConfig("ti2v5b_landscape", 256, 1, 31, 44, 80, 3, None),
    "ti2v5b_portrait": DecodeConfig("ti2v5b_portrait", 256, 1, 31, 80, 44, 4, None),
    "ti2v5b_landscape_b2": DecodeConfig("ti2v5b_landscape_b2", 256, 2, 31, 44, 80, 4, None),
}


@dataclass(frozen=True)
class ConvConfig:
    """A single causal 3x3x3 conv: x [B, C, t, h, w] with n_cache cached frames."""
    name: str
    C: int
    t: int
    h: int
    w: int
    n_cache: int
    seed: int

    def tensors(self):
        k = (self.C, self.C, 3, 3, 3)
        std = 1.0 / np.sqrt(fan_in(k))
        x = normal(self.seed, "x", (1, self.C, self.t, self.h, self.w))
        cache = normal(self.seed, "cache", (1, self.C, self.n_cache, self.h, self.w))
        return x, cache, normal(self.seed, "weight", k, std), normal(self.seed, "bias", (self.C,), std)


CONV_CONFIGS = {
    "conv1024_l0": ConvConfig("conv1024_l0", 1024, 1, 44, 80, 2, 1),
    "conv256_l3": ConvConfig("conv256_l3", 256, 4, 352, 640, 2, 1),
}


@dataclass(frozen=True)
class AttnConfig:
    """The mid-block attention block alone: x [B, C, T, h, w], attention over h*w per frame."""
    name: str
    C: int
    T: int
    h: int
    w: int
    seed: int

    def tensors(self):
        c = self.C
        std = 1.0 / np.sqrt(c)
        return {
            "x": normal(self.seed, "x", (1, c, self.T, self.h, self.w)),
            "gamma": normal(self.seed, "norm.gamma", (c, 1, 1), 0.1, 1.0),
            "qkv_w": normal(self.seed, "to_qkv.weight", (3 * c, c, 1, 1), std),
            "qkv_b": normal(self.seed, "to_qkv.bias", (3 * c,), std),
            "proj_w": normal(self.seed, "proj.weight", (c, c, 1, 1), std),
            "proj_b": normal(self.seed, "proj.bias", (c,), std),
        }


# attn1024_31f: the TI2V-5B mid block over 31 latent frames of 44x80. The *_s14400 configs:
# the Wan2.1 720p latent frame (90x160 = 14,400 positions per frame), with the block width a
# parameter (384, Wan2.1's mid-block width, and 1024): 2 frames for the parity tests, 21 (81
# video frames) for the measurement.
ATTN_CONFIGS = {
    "attn1024_31f": AttnConfig("attn1024_31f", 1024, 31, 44, 80, 2),
    "attn384_s14400": AttnConfig("attn384_s14400", 384, 2, 90, 160, 5),
    "attn1024_s14400": AttnConfig("attn1024_s14400", 1024, 2, 90, 160, 6),
    "attn384_s14400_21f": AttnConfig("attn384_s14400_21f", 384, 21, 90, 160, 5),
    "attn1024_s14400_21f": AttnConfig("attn1024_s14400_21f", 1024, 21, 90, 160, 6),
}
