"""Pins of the cached-KV prefill oracle (oracle/cached.py) against the plain
fp64 definition (the C oracle) and against what chunking must preserve."""
import numpy as np
import torch

import oracle
from oracle import cached


def _draw(B, S, Hq, Hkv, D, seed, dt=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, Hq, D, generator=g).to(dt)
    k = torch.randn(B, S, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, S, Hkv, D, generator=g).to(dt)
    return q, k, v


def test_empty_cache_is_the_plain_prefill():
    q, k, v = _draw(2, 37, 4, 2, 16, 0)
    for causal in (False, True):
        want = oracle.sdpa(q, k, v, scale=0.25, causal=causal)
        got = cached.prefill_cached(q, k[:, :0], v[:, :0], k, v, cache_len=0, scale=0.25, causal=causal)
        assert np.abs(got["out"] - want["out"]).max() < 1e-12
        assert np.abs(got["lse"] - want["lse"]).max() < 1e-12


def test_chunked_prefill_equals_the_whole_causal_prefill():
    """Chunk c of a sequence, with every earlier token as its cache, gives the
    rows the one-shot causal prefill gives for those queries."""
    q, k, v = _draw(1, 90, 6, 3, 32, 1)
    whole = oracle.sdpa(q, k, v, scale=0.2, causal=True)
    for lo, hi in ((0, 17), (17, 64), (64, 90)):
        got = cached.prefill_cached(q[:, lo:hi], k, v, k[:, lo:hi], v[:, lo:hi], cache_len=lo, scale=0.2,
                                    causal=True)
        assert np.abs(got["out"] - whole["out"][:, lo:hi]).max() < 1e-12
        assert np.abs(got["lse"] - whole["lse"][:, :, lo:hi]).max() < 1e-12


def test_full_attention_is_the_plain_definition_on_concatenated_keys():
    q, k, v = _draw(2, 40, 4, 1, 16, 2)
    kc, vc = _draw(2, 50, 1, 1, 16, 3)[1:]
    want = oracle.sdpa(q, torch.cat([kc[:, :33], k], 1), torch.cat([vc[:, :33], v], 1), scale=0.3, causal=False)
    got = cached.prefill_cached(q, kc, vc, k, v, cache_len=33, scale=0.3, causal=False)
    assert np.abs(got["out"] - want["out"]).max() < 1e-12


def test_cache_is_visible_to_every_query_and_slots_past_cache_len_are_not_keys():
    """Causal: query 0 of a chunk with as many queries as new keys sees the
    whole cache and new key 0 only; cache slots past cache_len (here huge
    values) never count."""
    q, k, v = _draw(1, 8, 2, 2, 16, 4)
    kc, vc = _draw(1, 12, 2, 2, 16, 5)[1:]
    kc[:, 5:] = 1e4
    vc[:, 5:] = float("nan")
    got = cached.prefill_cached(q, kc, vc, k, v, cache_len=5, scale=0.25, causal=True)
    want0 = oracle.sdpa(q[:, :1], torch.cat([kc[:, :5], k[:, :1]], 1), torch.cat([vc[:, :5], v[:, :1]], 1),
                        scale=0.25, causal=False)
    assert np.abs(got["out"][:, :1] - want0["out"]).max() < 1e-12
    assert not np.isnan(got["out"]).any()
    vis = cached.visible(8, 5, 8, True)
    assert vis[:, :5].all() and vis[0, 5:].sum() == 1 and vis[7, 5:].all()


def test_more_queries_than_new_keys_leaves_early_queries_the_cache_only():
    vis = cached.visible(6, 4, 3, True)
    assert vis[:, :4].all()
    assert vis[:3, 4:].sum() == 0 and vis[3, 4:].tolist() == [True, False, False]


def test_constant_values_and_single_visible_key():
    q, k, v = _draw(1, 4, 2, 1, 8, 6)
    kc, vc = _draw(1, 3, 1, 1, 8, 7)[1:]
    vc[:] = 0.5
    v[:] = 0.5
    got = cached.prefill_cached(q, kc, vc, k, v, cache_len=3, scale=1.0, causal=True)
    assert np.abs(got["out"] - 0.5).max() < 1e-12
    got = cached.prefill_cached(q[:, :1], kc, vc, k[:, :1], v[:, :1] * 3, cache_len=0, scale=1.0, causal=True)
    assert np.abs(got["out"][0, 0] - 1.5).max() < 1e-12
