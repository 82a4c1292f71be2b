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


def prefill_masked(q, k, v, mask, *, scale: float, causal: bool):
    """fp64 attention with a full additive mask added to the scaled scores:
    O = softmax(Q K^T * scale + mask [+ causal]) V, the mainloop's full-mask
    path ("Xe SDPA Forward Mainloop", sections "Runtime args / params" and
    "Compact shape table", row "Mask"; with causal it also applies the
    bottom-right causal rule).

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D|Dv]; mask [Bm, Hm, Sq, Sk] with Bm in
    {1, B} and Hm in {1, Hq} (broadcast), any float dtype (converted exactly).
    Returns {"out": [B, Sq, Hq, Dv] float64, "lse": [B, Hq, Sq]}; a row with no
    finite score gets O = 0 and lse = -inf.  Written out with torch float64
    matmuls on the CPU; no code shared with the other oracles."""
    import torch

    B, Sq, Hq, D = (int(s) for s in q.shape)
    Sk, Hkv, Dv = int(k.shape[1]), int(k.shape[2]), int(v.shape[-1])
    G = Hq // Hkv
    m64 = mask.to(torch.float64)
    qd, kd, vd = q.to(torch.float64), k.to(torch.float64), v.to(torch.float64)
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        cm = torch.where(j <= i + (Sk - Sq), 0.0, float("-inf")).to(torch.float64)
    out = np.zeros((B, Sq, Hq, Dv), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s = (qd[b, :, h] @ kd[b, :, h // G].T) * scale + m64[b % m64.shape[0], h % m64.shape[1]]
            if causal:
                s = s + cm
            mx = s.max(dim=1, keepdim=True).values
            has = torch.isfinite(mx)
            e = torch.where(has, torch.exp(s - torch.where(has, mx, torch.zeros_like(mx))), torch.zeros_like(s))
            den = e.sum(dim=1, keepdim=True)
            safe = torch.where(den > 0, den, torch.ones_like(den))
            out[b, :, h] = torch.where(den > 0, (e @ vd[b, :, h // G]) / safe, torch.zeros(1)).numpy()
            lse[b, h] = torch.where(den[:, 0] > 0, mx[:, 0] + torch.log(safe[:, 0]), float("-inf")).numpy()
    return {"out": out, "lse": lse}
