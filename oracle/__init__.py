"""fp64 CPU oracle of the Spatial-Transformer (Transformer2DModel) block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library
under ``latent_diffusion_net_amd/`` never imports it and shares no code with it.

``oracle.block``  vectorised float64 NumPy/SciPy implementation of the block
                  (with the cross-attention key mask)
``oracle.unet``   SiLU, 3x3 convolution, ResnetBlock2D, classifier-free
                  guidance and the DDPM step, float64
``oracle.brute``  scalar-loop implementation for tiny shapes (stdlib only)
"""
from .block import (attention, block_forward, from_tokens, gelu_erf, geglu,
                    group_norm, layer_norm, linear, to_tokens)

__all__ = ["attention", "block_forward", "from_tokens", "gelu_erf", "geglu",
           "group_norm", "layer_norm", "linear", "to_tokens"]
