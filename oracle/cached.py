"""Cached-KV (chunked) prefill -- TEST INFRASTRUCTURE (oracle side).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU leg may
use this module; the HIP path never does.

The page "Xe SDPA Forward Mainloop -- Key Loops + Shapes" runs a cached mode
in which the key sequence is a cached prefix of seq_len_kv_cache keys (held
in their own tensors) followed by the chunk's new keys: the first
ceil(seq_len_kv_cache / block) K blocks come from the cache, the rest from
the new tensors, indexed from the first new key (sections "Startup prefetch +
init" and "Outer K-block loop", and the K prefetch of the mainloop body),
and the causal mask is applied only to blocks that are not cache blocks
(section "mask branches").  Reading taken here: every query sees every cached
key; query i sees new key j iff j <= i + new_len - q_len (the bottom-right
rule of the plain prefill, on the new keys); a cache block's slots past
seq_len_kv_cache hold no key.

The definition is written out directly in fp64 (torch float64 matmuls on the
CPU as the only library steps): scores over the concatenated keys, the mask
above, a max-subtracted softmax, the weighted sum of values.  It shares no
code with the C oracle or the HIP path.
"""
from __future__ import annotations

import numpy as np


def visible(q_len: int, cache_len: int, new_len: int, causal: bool):
    """Boolean [q_len, cache_len + new_len]: key t is visible to query i."""
    vis = np.ones((q_len, cache_len + new_len), dtype=bool)
    if causal:
        i = np.arange(q_len)[:, None]
        j = np.arange(new_len)[None, :]
        vis[:, cache_len:] = j <= i + (new_len - q_len)
    return vis


def _f64(x):
    import torch

    return x.to(torch.float64) if isinstance(x, torch.Tensor) else torch.as_tensor(np.asarray(x, np.float64))


def prefill_cached(q, k_cache, v_cache, k, v, *, cache_len: int, scale: float, causal: bool):
    """fp64 attention of the chunk's queries over cache keys 0 .. cache_len-1
    followed by the chunk's own keys.

    q [B, Sq, Hq, D]; k_cache/v_cache [B, >= cache_len, Hkv, D|Dv];
    k/v [B, new_len, Hkv, D|Dv].  Query head h reads KV head h / (Hq / Hkv).
    Returns {"out": [B, Sq, Hq, Dv] float64, "lse": [B, Hq, Sq] (natural
    log)}; a query with no visible key gets O = 0 and lse = -inf.
    """
    import torch

    B, Sq, Hq, D = (int(s) for s in q.shape)
    new_len, Hkv = int(k.shape[1]), int(k.shape[2])
    Dv = int(v.shape[-1])
    G = Hq // Hkv
    keys = torch.cat([_f64(k_cache[:, :cache_len]), _f64(k)], dim=1)      # [B, T, Hkv, D]
    vals = torch.cat([_f64(v_cache[:, :cache_len]), _f64(v)], dim=1)
    vis = torch.as_tensor(visible(Sq, cache_len, new_len, causal))
    qd = _f64(q)
    out = np.zeros((B, Sq, Hq, Dv), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kh = keys[b, :, h // G]                     # [T, D]
            vh = vals[b, :, h // G]                     # [T, Dv]
            s = (qd[b, :, h] @ kh.T) * scale            # [Sq, T]
            s = s.masked_fill(~vis, float("-inf"))
            m = s.max(dim=1, keepdim=True).values
            has = torch.isfinite(m)
            e = torch.where(has, torch.exp(s - torch.where(has, m, torch.zeros_like(m))), torch.zeros_like(s))
            den = e.sum(dim=1, keepdim=True)
            o = torch.where(den > 0, (e @ vh) / torch.where(den > 0, den, torch.ones_like(den)), torch.zeros(1))
            out[b, :, h] = o.numpy()
            lse[b, h] = torch.where(den[:, 0] > 0, m[:, 0] + torch.log(den[:, 0]), float("-inf")).numpy()
    return {"out": out, "lse": lse}
