"""The blocked online-softmax algorithm with split-KV combine (pages' method,
fp64) reproduces the plain two-pass definition computed by the C oracle."""
import math

import numpy as np
import pytest

from oracle import blocked


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_k", [1, 7, 64])
@pytest.mark.parametrize("num_splits", [1, 3, 16])
@pytest.mark.parametrize("sq,sk", [(9, 23), (23, 9), (1, 40), (16, 16)])
def test_online_equals_two_pass(oracle_mod, causal, block_k, num_splits, sq, sk):
    hq, hkv, d, dv = 4, 2, 8, 5
    q = _rand((1, sq, hq, d), 1 + sq)
    k = _rand((1, sk, hkv, d), 2 + sk)
    v = _rand((1, sk, hkv, dv), 3 + sk)
    scale = 1.0 / math.sqrt(d)
    ref = oracle_mod.sdpa(q, k, v, scale=scale, causal=causal)
    out, lse = blocked.attention_blocked(q[0], k[0], v[0], scale=scale, causal=causal, block_k=block_k,
                                         num_splits=num_splits, group=hq // hkv)
    assert not np.isnan(out).any()
    np.testing.assert_allclose(out, ref["out"][0], rtol=0, atol=1e-12)
    fin = np.isfinite(ref["lse"][0])
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], ref["lse"][0][fin], rtol=0, atol=1e-12)


def test_scale_zero_and_empty_splits(oracle_mod):
    q = _rand((1, 5, 2, 4), 9)
    k = _rand((1, 3, 1, 4), 10)
    v = _rand((1, 3, 1, 4), 11)
    ref = oracle_mod.sdpa(q, k, v, scale=0.0, causal=True)
    out, lse = blocked.attention_blocked(q[0], k[0], v[0], scale=0.0, causal=True, block_k=1, num_splits=16,
                                         group=2)
    np.testing.assert_allclose(out, ref["out"][0], atol=1e-14)
    assert (out[:2] == 0).all() and np.isneginf(lse[:, :2]).all()
