"""Blocked online-softmax attention with split-KV combine, fp64 numpy.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  This is the *algorithm* the
pages describe, written out step by step so that tests can show it reproduces
the plain definition in ``sdpa_oracle.c`` (the online rescale is an identity in
exact arithmetic).  It is slow and meant for small shapes.

Steps follow "Xe SDPA Forward Mainloop -- Key Loops + Shapes":
  * section "Arguments / params": the softmax scale is multiplied by log2(e)
    once so that every exponential is a base-2 exponential;
  * section "Full simplified pseudocode" (the per-K-block loop): scores of one
    key block, mask, block row max, new running max, rescale factor
    2^(old_max - new_max), probabilities 2^(scale*S - new_max), running sum
    rescaled and incremented, output accumulator rescaled and incremented by
    P @ V_block;
  * section "Outer K-block loop": one work item owns the block range
    [blk_k0, blk_k1); splitting the key range this way gives the partial
    results that the two-phase decode of "xe2-sdp-kernels" (section "Assets")
    combines in its second phase.
The combine rescales each split by 2^(m_s - M) with M the largest split max,
the same rescale the online loop applies between blocks.  The final division by
the running sum is the plain normalisation the mainloop pages leave to the
epilogue.  Empty splits (max = -inf) get weight 0; a row with no visible key at
all returns 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def _visible(i: int, j: np.ndarray, sq: int, sk: int, causal: bool) -> np.ndarray:
    """Bottom-right causal rule: key j visible to query i iff j <= i + sk - sq."""
    if not causal:
        return j < sk
    return j <= i + sk - sq


def split_partials(q, k, v, scale, causal, block_k, k_begin, k_end):
    """Online softmax over keys [k_begin, k_end) for every query row of one head.

    q: [Sq, D], k: [Sk, D], v: [Sk, Dv] float64.  Returns the unnormalised
    accumulator O_s [Sq, Dv], the running max m_s [Sq] (base-2 scaled domain)
    and the running sum l_s [Sq].
    """
    sq, sk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    s2 = scale * LOG2E                      # scale folded with log2(e)
    o = np.zeros((sq, dv))
    m = np.full(sq, -np.inf)
    l = np.zeros(sq)
    rows = np.arange(sq)
    for kb in range(k_begin, k_end, block_k):
        ke = min(kb + block_k, k_end)
        cols = np.arange(kb, ke)
        t = s2 * (q @ k[kb:ke].T)           # scores in the base-2 scaled domain [Sq, BK]
        vis = np.stack([_visible(i, cols, sq, sk, causal) for i in rows]) if sq else np.zeros((0, ke - kb), bool)
        # mask after scaling: the same as masking raw scores for scale > 0, and
        # free of 0 * (-inf) when scale == 0
        t = np.where(vis, t, -np.inf)
        bmax = t.max(axis=1) if t.shape[1] else np.full(sq, -np.inf)
        new_m = np.maximum(m, bmax)
        # rows whose running max is still -inf have seen no visible key yet:
        # use 0 as the subtrahend so that no (-inf) - (-inf) appears
        safe_m = np.where(np.isfinite(new_m), new_m, 0.0)
        alpha = np.exp2(np.where(np.isfinite(m), m - safe_m, -np.inf))
        p = np.exp2(t - safe_m[:, None])
        p = np.where(vis, p, 0.0)
        l = l * alpha + p.sum(axis=1)
        o = o * alpha[:, None] + p @ v[kb:ke]
        m = new_m
    return o, m, l


def combine(o_parts, m_parts, l_parts):
    """Second phase: merge split partials (lists over splits) into O and lse."""
    m_all = np.stack(m_parts)               # [S, Sq]
    big = m_all.max(axis=0)
    safe = np.where(np.isfinite(big), big, 0.0)
    w = np.exp2(np.where(np.isfinite(m_all), m_all - safe, -np.inf))   # [S, Sq]
    num = sum(w[s][:, None] * o_parts[s] for s in range(len(o_parts)))
    den = sum(w[s] * l_parts[s] for s in range(len(l_parts)))
    out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
    lse = np.where(den > 0, (big + np.log2(np.where(den > 0, den, 1.0))) / LOG2E, -np.inf)
    return out, lse


def attention_blocked(q, k, v, *, scale, causal, block_k=64, num_splits=1, group=1):
    """Blocked online attention for q [Sq, Hq, D], k [Sk, Hkv, D], v [Sk, Hkv, Dv]
    (one batch entry, float64).  The key range is cut into ``num_splits``
    contiguous ranges of equal block count (trailing ranges may be empty),
    each processed with ``split_partials`` and merged with ``combine``.
    Returns (out [Sq, Hq, Dv], lse [Hq, Sq])."""
    sq, hq, _ = q.shape
    sk = k.shape[0]
    dv = v.shape[2]
    out = np.zeros((sq, hq, dv))
    lse = np.zeros((hq, sq))
    n_blocks = -(-sk // block_k) if sk else 0
    per_split = -(-n_blocks // num_splits) if n_blocks else 0
    for h in range(hq):
        g = h // group
        parts = []
        for s in range(num_splits):
            k0 = min(s * per_split * block_k, sk)
            k1 = min((s + 1) * per_split * block_k, sk)
            parts.append(split_partials(q[:, h], k[:, g], v[:, g], scale, causal, block_k, k0, k1))
        o, ls = combine([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        out[:, h] = o
        lse[h] = ls
    return out, lse
