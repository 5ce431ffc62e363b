"""CPU oracle of the Wan2.2 TI2V-5B VAE decoder (test infrastructure).

This package is test infrastructure, not part of the product. Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import,
call or execute anything under ``oracle/``. The HIP library and its Python
binding never import it, and it imports nothing from them. Its only shared
dependency is the seeded input generator in ``synthetic/``.

It is a plain, slow numpy implementation of what FastVideo's
"wan22_vae_decode reference.py" page defines (sections "What is computed",
"The parts", "The first latent frame yields one frame", "Causal caches",
"Precision"), run chunk by chunk with the causal caches, in three modes:

* ``fp64``: every value in float64, no rounding (ground truth);
* ``fp32``: every stored value rounded to float32 where the page's float32
  decode produces it;
* ``bf16``: every stored value rounded to bfloat16 (round to nearest even) at
  the rounding points the page's "Precision" section lists for the bf16
  decode.

Sums inside a convolution, matmul or softmax are accumulated in float64 unless
``acc="f32"`` is passed (allowed for the full-size configurations, where the
page itself says the bf16 and fp32 kernels accumulate in float32).

``tiled.py`` holds the spatially tiled decode of the diffusers PR page on Wan
tiling, with the blend rule read as its module docstring says.

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_ops.py``, ``tests/test_oracle_decoder.py`` or
``tests/test_oracle_tiled.py`` against brute force, a library routine, a closed
form or an invariant the pages state.
"""
from .decoder import (  # noqa: F401
    MODES,
    Prec,
    attention,
    attention_rows,
    cached_conv,
    causal_conv,
    conv_points,
    decode,
    decode_chunk,
    dup_up,
    psnr,
    residual_block,
    rms_norm,
    round_bf16,
    silu,
    spatial_upsample,
    time_upsample,
    unpatchify,
)
from .tiled import compose, decode_tiled, tile_grid  # noqa: F401
