"""MI355X-native Spatial-Transformer (Transformer2DModel) block.

The compute path is ``libst_block.so`` (hand-written HIP for gfx950, C ABI in
``include/st_block.h``); this package only marshals arguments to it.
"""
from .binding import (EXPORTS, KERNEL_KINDS, STBlock, STError, STResnet, STUNet,
                      array_to_device, last_error, load_library, params_to_device,
                      tree_to_device)

__all__ = ["EXPORTS", "KERNEL_KINDS", "STBlock", "STError", "STResnet", "STUNet",
           "array_to_device", "last_error", "load_library", "params_to_device",
           "tree_to_device"]
