"""FlashMask masked-attention forward pass for AMD Instinct MI355X (gfx950).

The computation lives in libflashmask.so (HIP kernels behind a C ABI,
include/flashmask.h); :mod:`masked_attention_fm_amd.flashmask` is its thin
ctypes binding.  :mod:`masked_attention_fm_amd.inputs` draws the seeded
synthetic workloads.
"""
from .flashmask import (FlashMaskError, fm_attn_fwd, fm_attn_tile_shape, fm_classify_tiles,
                        fm_profile_enable, fm_profile_read, fm_set_option, fm_tile_schedule)

__all__ = ["FlashMaskError", "fm_attn_fwd", "fm_attn_tile_shape", "fm_classify_tiles",
           "fm_profile_enable", "fm_profile_read", "fm_set_option", "fm_tile_schedule"]
