"""Boolean -> additive mask conversion -- TEST INFRASTRUCTURE (oracle side).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU leg may
use this module; the HIP path never does.

The page "Xe SDPA Forward Mainloop -- Key Loops + Shapes" gives the mainloop
an optional full mask among its runtime arguments (section "Runtime args /
params") that the mask step applies to the score tile (section "Compact
shape table", row "Mask"); the page "xe2-sdp-kernels" names a memory-bound
mask_convert kernel (section "Performance testing").  Neither fixes the
encodings.  Reading taken here: the input is one byte per (query, key)
element, nonzero meaning the key takes part in the query's attention; the
output is the additive mask in a 16-bit float type, 0 where the key takes
part and -inf where it does not, element for element in the same order.
"""
from __future__ import annotations

import numpy as np


def mask_convert(mask, out_dtype: str):
    """Additive mask (numpy float16 for "f16"; for "bf16" the uint16 bit
    patterns, as numpy has no bfloat16) of a uint8 mask of any shape."""
    keep = np.asarray(mask, dtype=np.uint8) != 0
    if out_dtype == "f16":
        return np.where(keep, np.float16(0.0), np.float16(-np.inf)).astype(np.float16)
    if out_dtype == "bf16":
        # bfloat16 is the upper half of an IEEE float32: +0 -> 0x0000, -inf -> 0xff80
        bits = (np.array([0.0, -np.inf], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return np.where(keep, bits[0], bits[1]).astype(np.uint16)
    raise ValueError(out_dtype)
