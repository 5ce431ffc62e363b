"""MI355X (gfx950) Wan2.2 TI2V-5B VAE decoder.

The decoder runs in libwanvae.so (hand-written HIP kernels behind the C ABI of
include/wanvae.h); this package is its Python binding.
"""
from .wanvae import (  # noqa: F401
    BF16,
    F32,
    NCTHW,
    NTHWC,
    WanVAEError,
    attn_block,
    causal_conv3d,
    decode,
    decode_workspace_size,
    lib,
    wanvae_attn_block,
    wanvae_causal_conv3d,
    wanvae_decode,
)
