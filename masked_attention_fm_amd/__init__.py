"""FlashMask masked-attention forward pass for AMD Instinct MI355X (gfx950).

The computation lives in libflashmask.so (HIP kernels behind a C ABI,
include/flashmask.h); :mod:`masked_attention_fm_amd.flashmask` is its thin
ctypes binding.  :mod:`masked_attention_fm_amd.masks` writes mask
specifications (per call, per head, per layer) down as the interval arrays the
library takes; :mod:`masked_attention_fm_amd.inputs` draws the seeded
synthetic workloads.
"""
from .flashmask import (FlashMaskError, fm_attn_bwd, fm_attn_bwd_multi, fm_attn_bwd_per_head, fm_attn_fwd,
                        fm_attn_fwd_fp8, fm_attn_fwd_multi, fm_attn_fwd_per_head, fm_attn_tile_shape,
                        fm_classify_tiles, fm_classify_tiles_multi, fm_profile_enable, fm_profile_read,
                        fm_set_option, fm_tile_schedule, fm_tile_schedule_multi)
from .masks import (Causal, Documents, Full, PrefixLM, Ranges, SinksWindow, SlidingWindow, head_intervals,
                    layer_intervals, mask_intervals)

__all__ = ["FlashMaskError", "fm_attn_bwd", "fm_attn_bwd_multi", "fm_attn_bwd_per_head", "fm_attn_fwd",
           "fm_attn_fwd_fp8", "fm_attn_fwd_multi", "fm_attn_fwd_per_head", "fm_attn_tile_shape",
           "fm_classify_tiles", "fm_classify_tiles_multi", "fm_profile_enable", "fm_profile_read",
           "fm_set_option", "fm_tile_schedule", "fm_tile_schedule_multi", "Causal", "Documents", "Full",
           "PrefixLM", "Ranges", "SinksWindow", "SlidingWindow", "head_intervals", "layer_intervals",
           "mask_intervals"]
