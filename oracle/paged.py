"""Paged and variable-length KV decode -- TEST INFRASTRUCTURE (oracle side).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU leg may
use this module; the HIP path never does.

The page "Xe SDPA Forward Mainloop -- Key Loops + Shapes" lists optional
paged-KV metadata among the mainloop's runtime arguments (section "Runtime
args / params": a page table pointer, a page size and per-sequence page
counts) and a helper that maps a logical K tile to its physical tile
(section "Helpers", get_physical_k_tile()); the launcher's runtime variant
also selects a variable-length mode (section "Launcher -> kernel", isVarLen).
The pages do not spell the layout out.  Reading taken here: the key (and
value) cache is a pool of physical pages shaped [num_pages, page_size, H_kv,
D]; logical page p of sequence b (keys p*page_size .. (p+1)*page_size - 1)
is physical page page_table[b, p]; sequence b holds seq_lens[b] keys.

The oracle gathers each sequence's keys in logical order -- plain indexing,
none of the method's arithmetic -- and evaluates the fp64 definition of
``oracle.sdpa`` on them.
"""
from __future__ import annotations

import numpy as np

from . import sdpa


def gather_sequence(cache, page_table, page_size: int, seq_len: int, b: int):
    """Keys (or values) 0 .. seq_len-1 of sequence b, in logical order:
    [seq_len, H_kv, D] from a paged cache, or the first seq_len rows of
    cache[b] when page_table is None (contiguous [B, kv_len, H_kv, D])."""
    import torch

    if page_table is None:
        return cache[b, :seq_len]
    keys = torch.arange(seq_len)
    pages = torch.as_tensor(np.asarray(page_table))[b, keys // page_size].long()
    slots = keys % page_size
    return cache[pages, slots]


def decode_paged(q, k_cache, v_cache, *, page_table, page_size: int, seq_lens, scale: float, kv_len=None):
    """fp64 decode (one query token per sequence) over paged and/or
    variable-length keys.

    q: [B, Hq, D]; k_cache/v_cache: [num_pages, page_size, Hkv, D|Dv] when
    page_table ([B, pages_per_seq] ints) is given, else [B, kv_len, Hkv, ...];
    seq_lens: [B] ints, or None for kv_len keys in every sequence, kv_len
    defaulting to what a sequence can hold: the dense cache's length, or a
    full table row (pages_per_seq * page_size).
    Returns {"out": [B, Hq, Dv] float64, "lse": [B, Hq]} with O = 0 and
    lse = -inf for a sequence without keys.
    """
    import torch

    B, Hq, D = (int(s) for s in q.shape)
    Dv = int(v_cache.shape[-1])
    if seq_lens is None:
        if kv_len is None:
            kv_len = (int(k_cache.shape[1]) if page_table is None
                      else int(np.asarray(page_table).shape[1]) * page_size)
        seq_lens = [int(kv_len)] * B
    out = np.zeros((B, Hq, Dv), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        kb = gather_sequence(k_cache, page_table, page_size, n, b)
        vb = gather_sequence(v_cache, page_table, page_size, n, b)
        if isinstance(kb, torch.Tensor):
            kb, vb = kb.contiguous(), vb.contiguous()
        r = sdpa(q[b:b + 1].reshape(1, 1, Hq, D), kb[None], vb[None], scale=scale, causal=False)
        out[b] = r["out"][0, 0]
        lse[b] = r["lse"][0, :, 0]
    return {"out": out, "lse": lse}
