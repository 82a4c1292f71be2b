"""MI355X-native fused scaled-dot-product-attention forward.

Python front end of the C-ABI library ``libsdpa_mi355x.so`` (see
``include/sdpa.h``): ``prefill`` (causal or full, GQA), ``prefill_cached`` (a
chunk over a cached prefix), ``prefill_masked`` (a full additive mask),
``decode`` (two-phase split-KV), ``decode_paged`` (variable-length and paged
caches), ``mask_convert`` (boolean to additive masks) and the host planner
``plan``.  The compute runs in hand-written HIP
kernels for gfx950; PyTorch only provides device memory and streams.
"""
from .binding import (  # noqa: F401
    BF16,
    F16,
    FP8_E4M3,
    Plan,
    Problem,
    SdpaError,
    decode,
    decode_noalloc,
    decode_paged,
    decode_workspace,
    hbm_read_probe,
    load,
    loop_counts,
    make_problem,
    mask_convert,
    plan,
    prefill,
    prefill_cached,
    prefill_cached_workspace_bytes,
    prefill_masked,
    prefill_workspace_bytes,
    set_prefill_variant,
)

__all__ = ["prefill", "prefill_workspace_bytes", "prefill_cached", "prefill_cached_workspace_bytes", "prefill_masked", "decode", "decode_noalloc", "decode_paged", "decode_workspace", "hbm_read_probe", "mask_convert", "plan",
           "loop_counts", "set_prefill_variant", "make_problem", "load", "Problem", "Plan", "SdpaError", "F16", "BF16", "FP8_E4M3"]
