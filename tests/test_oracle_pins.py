"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself: exact dtype decoding by
torch, closed forms, invariants, special cases that reduce to library routines
(torch's float64 scaled_dot_product_attention, numpy mean/argmax, scipy
expit/logsumexp), and the blocked online algorithm of the pages.  Each case is
chosen so that a plausible mistake (dropped scale, wrong sign, transposed
operand, wrong GQA index, wrong causal offset, NaN on empty rows) fails it.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit, logsumexp

from attention_flash_sdpa_amd import inputs

pytestmark = []


def _rand(shape, seed, dtype=np.float64):
    return np.random.default_rng(seed).standard_normal(shape).astype(dtype)


def _torch_ref(q, k, v, scale, causal):
    """torch float64 SDPA with an explicit bottom-right mask; rows with no
    visible key are returned as NaN (torch's own behaviour) and skipped by
    callers."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    if causal:
        mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
    else:
        mask = torch.ones(Sq, Sk, dtype=torch.bool)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy(), mask.numpy()


# ---------------------------------------------------------------- dtype decoding
def test_decode_bf16_f16_all_patterns(oracle_mod):
    """Every bf16 / fp16 bit pattern widens exactly as torch widens it."""
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    for tdt, code in ((torch.bfloat16, oracle_mod.BF16), (torch.float16, oracle_mod.F16)):
        want = bits.view(tdt).to(torch.float64).numpy()
        got = np.array([oracle_mod.decode_scalar(code, b) for b in range(65536)])
        assert np.array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok])
        # the same widening on the attention path: one key, so O equals V
        v = bits.view(tdt)[::97].reshape(1, 1, 1, -1).contiguous()
        z = torch.zeros(1, 1, 1, 1, dtype=tdt)
        out = oracle_mod.sdpa(z, z, v, scale=1.0, causal=False)["out"].reshape(-1)
        ref = v.to(torch.float64).reshape(-1).numpy()
        fin = np.isfinite(ref)
        assert np.array_equal(out[fin], ref[fin])


def test_decode_e4m3_all_patterns(oracle_mod):
    bits = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    want = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.decode_scalar(oracle_mod.FP8_E4M3, b) for b in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


# ---------------------------------------------------------------- closed forms
def test_two_key_closed_form(oracle_mod):
    """Sq=1, Sk=2: O = v0 + expit(s1 - s0) (v1 - v0), lse = logaddexp(s0, s1)."""
    q = _rand((1, 1, 1, 5), 1)
    k = _rand((1, 2, 1, 5), 2)
    v = _rand((1, 2, 1, 3), 3)
    scale = 0.37
    s0 = scale * float(q[0, 0, 0] @ k[0, 0, 0])
    s1 = scale * float(q[0, 0, 0] @ k[0, 1, 0])
    want = v[0, 0, 0] + expit(s1 - s0) * (v[0, 1, 0] - v[0, 0, 0])
    res = oracle_mod.sdpa(q, k, v, scale=scale, causal=False)
    np.testing.assert_allclose(res["out"][0, 0, 0], want, rtol=0, atol=1e-14)
    assert abs(res["lse"][0, 0, 0] - np.logaddexp(s0, s1)) < 1e-14


def test_scale_zero_is_mean_and_lse_is_log_count(oracle_mod):
    q = _rand((2, 6, 4, 8), 4)
    k = _rand((2, 9, 2, 8), 5)
    v = _rand((2, 9, 2, 3), 6)
    res = oracle_mod.sdpa(q, k, v, scale=0.0, causal=True)
    off = 9 - 6
    for b in range(2):
        for i in range(6):
            n = i + off + 1
            for h in range(4):
                np.testing.assert_allclose(res["out"][b, i, h], v[b, :n, h // 2].mean(axis=0), atol=1e-14)
                assert abs(res["lse"][b, h, i] - math.log(n)) < 1e-14


def test_single_key_returns_v0(oracle_mod):
    q = _rand((1, 3, 2, 16), 7)
    k = _rand((1, 1, 1, 16), 8)
    v = _rand((1, 1, 1, 16), 9)
    res = oracle_mod.sdpa(q, k, v, scale=0.25, causal=False)
    for i in range(3):
        for h in range(2):
            assert np.array_equal(res["out"][0, i, h], v[0, 0, 0])


def test_large_logits_give_argmax_row(oracle_mod):
    """Scores scaled by 1e3 make the softmax one-hot; the max subtraction must
    keep exp from overflowing."""
    q = _rand((1, 4, 1, 8), 10) * 1e3
    k = _rand((1, 6, 1, 8), 11)
    v = _rand((1, 6, 1, 5), 12)
    res = oracle_mod.sdpa(q, k, v, scale=1.0, causal=False)
    assert np.isfinite(res["out"]).all()
    for i in range(4):
        j = int(np.argmax(q[0, i, 0] @ k[0, :, 0].T))
        np.testing.assert_allclose(res["out"][0, i, 0], v[0, j, 0], atol=1e-12)


def test_constant_v_rows_return_the_constant(oracle_mod):
    q = _rand((1, 5, 2, 8), 13)
    k = _rand((1, 7, 1, 8), 14)
    c = _rand((4,), 15)
    v = np.broadcast_to(c, (1, 7, 1, 4)).copy()
    res = oracle_mod.sdpa(q, k, v, scale=0.5, causal=True)
    for i in range(5):
        for h in range(2):
            np.testing.assert_allclose(res["out"][0, i, h], c, atol=1e-14)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 4, 2, 2, 3, 3), (2, 3, 7, 4, 2, 5, 6), (1, 7, 5, 2, 1, 4, 4)])
def test_probability_rows_sum_to_one(oracle_mod, causal, shape):
    B, Sq, Sk, Hq, Hkv, D, Dv = shape
    q = _rand((B, Sq, Hq, D), 16)
    k = _rand((B, Sk, Hkv, D), 17)
    v = _rand((B, Sk, Hkv, Dv), 18)
    res = oracle_mod.sdpa(q, k, v, scale=1 / math.sqrt(D), causal=causal, want_probs=True)
    p = res["probs"]
    for i in range(Sq):
        n_vis = min(Sk, i + Sk - Sq + 1) if causal else Sk
        n_vis = max(n_vis, 0)
        row = p[:, i]                                      # [B, Hq, Sk]
        assert (row[..., n_vis:] == 0).all()               # masked keys carry no weight
        if n_vis > 0:
            np.testing.assert_allclose(row.sum(-1), 1.0, atol=1e-12)
            # lse consistency: p_ij = exp(s_ij - lse_i)
            assert (row[..., :n_vis] > 0).all()
        else:
            assert (res["out"][:, i] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 2, 1, 1, 1, 1), (1, 4, 4, 2, 1, 4, 4), (2, 3, 4, 4, 2, 3, 2),
                                   (1, 5, 9, 6, 3, 7, 5), (2, 9, 6, 4, 4, 8, 8)])
def test_matches_torch_float64_sdpa(oracle_mod, causal, shape):
    """Library routine: torch's float64 SDPA with an explicit bottom-right mask
    and K/V repeated per query head (GQA = MHA with repeat_interleave)."""
    B, Sq, Sk, Hq, Hkv, D, Dv = shape
    q = _rand((B, Sq, Hq, D), 20 + Sq)
    k = _rand((B, Sk, Hkv, D), 21 + Sk)
    v = _rand((B, Sk, Hkv, Dv), 22 + Dv)
    scale = 1.0 / math.sqrt(D) * 1.3
    res = oracle_mod.sdpa(q, k, v, scale=scale, causal=causal)
    ref, mask = _torch_ref(q, k, v, scale, causal)
    nonempty = mask.any(axis=1)                            # [Sq]
    np.testing.assert_allclose(res["out"][:, nonempty], ref[:, nonempty], rtol=0, atol=1e-12)
    assert (res["out"][:, ~nonempty] == 0).all()
    assert np.isneginf(res["lse"][:, :, ~nonempty]).all()
    # lse against scipy's logsumexp of torch-computed scores
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=2)
    for b in range(B):
        for h in range(Hq):
            s = scale * np.einsum("id,jd->ij", q[b, :, h], kk[b, :, h])
            for i in np.nonzero(nonempty)[0]:
                want = logsumexp(s[i][mask[i]])
                assert abs(res["lse"][b, h, i] - want) < 1e-12


def test_gqa_equals_repeated_mha(oracle_mod):
    q = _rand((1, 6, 8, 4), 30)
    k = _rand((1, 5, 2, 4), 31)
    v = _rand((1, 5, 2, 3), 32)
    a = oracle_mod.sdpa(q, k, v, scale=0.5, causal=False)["out"]
    b = oracle_mod.sdpa(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), scale=0.5, causal=False)["out"]
    np.testing.assert_allclose(a, b, atol=1e-14)
    # and differs from the wrong (h % Hkv) grouping
    kw = np.tile(k, (1, 1, 4, 1))
    vw = np.tile(v, (1, 1, 4, 1))
    c = oracle_mod.sdpa(q, kw, vw, scale=0.5, causal=False)["out"]
    assert np.abs(a - c).max() > 1e-3


def test_key_permutation_invariance_full_mask(oracle_mod):
    q = _rand((1, 4, 2, 6), 33)
    k = _rand((1, 11, 1, 6), 34)
    v = _rand((1, 11, 1, 5), 35)
    perm = np.random.default_rng(36).permutation(11)
    a = oracle_mod.sdpa(q, k, v, scale=0.4, causal=False)["out"]
    b = oracle_mod.sdpa(q, k[:, perm], v[:, perm], scale=0.4, causal=False)["out"]
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_linear_in_v(oracle_mod):
    q = _rand((1, 4, 2, 6), 37)
    k = _rand((1, 8, 2, 6), 38)
    v1 = _rand((1, 8, 2, 5), 39)
    v2 = _rand((1, 8, 2, 5), 40)
    f = lambda v: oracle_mod.sdpa(q, k, v, scale=0.4, causal=True)["out"]
    np.testing.assert_allclose(f(2.0 * v1 - 3.0 * v2), 2.0 * f(v1) - 3.0 * f(v2), atol=1e-13)


def test_causal_structure(oracle_mod):
    """Sq == Sk causal is lower-triangular (row 0 sees only key 0); causal with
    q_len == 1 equals the full mask; q_len > kv_len leaves the first rows empty."""
    q = _rand((1, 6, 1, 4), 41)
    k = _rand((1, 6, 1, 4), 42)
    v = _rand((1, 6, 1, 3), 43)
    r = oracle_mod.sdpa(q, k, v, scale=0.5, causal=True, want_probs=True)
    assert np.array_equal(r["out"][0, 0, 0], v[0, 0, 0])
    assert np.array_equal(r["probs"][0, :, 0] > 0, np.tril(np.ones((6, 6), bool)))
    a = oracle_mod.sdpa(q[:, :1], k, v, scale=0.5, causal=True)["out"]
    b = oracle_mod.sdpa(q[:, :1], k, v, scale=0.5, causal=False)["out"]
    assert np.array_equal(a, b)
    # tiny causal workload shape: q_len = 7 against kv_len = 5
    w = inputs.WORKLOADS["tiny_causal_bf16"]
    qq, kk, vv, _ = inputs.make_qkv(w)
    res = oracle_mod.sdpa(qq, kk, vv, scale=w.scale, causal=True)
    assert (res["out"][:, :2] == 0).all() and np.isneginf(res["lse"][:, :, :2]).all()
    assert np.isfinite(res["out"]).all()
    for b in range(w.batch):
        for h in range(w.head_q):
            assert np.array_equal(res["out"][b, 2, h], vv[b, 0, h // 7].double().numpy())
    assert w.valid_pairs() == 15


def test_empty_key_range_and_empty_queries(oracle_mod):
    q = _rand((1, 3, 2, 4), 44)
    k = np.zeros((1, 0, 1, 4))
    v = np.zeros((1, 0, 1, 4))
    r = oracle_mod.sdpa(q, k, v, scale=0.5, causal=False)
    assert (r["out"] == 0).all() and np.isneginf(r["lse"]).all()
    r = oracle_mod.sdpa(q[:, :0], _rand((1, 3, 1, 4), 45), _rand((1, 3, 1, 4), 46), scale=0.5, causal=True)
    assert r["out"].shape == (1, 0, 2, 4)


def test_rows_subset_matches_full(oracle_mod):
    q = _rand((2, 5, 4, 8), 47)
    k = _rand((2, 7, 2, 8), 48)
    v = _rand((2, 7, 2, 6), 49)
    full = oracle_mod.sdpa(q, k, v, scale=0.3, causal=True)
    rows = np.array([[1, 4, 3], [0, 0, 0], [1, 2, 1]])
    sub = oracle_mod.sdpa(q, k, v, scale=0.3, causal=True, rows=rows)
    for n, (b, i, h) in enumerate(rows):
        assert np.array_equal(sub["out"][n], full["out"][b, i, h])
        assert sub["lse"][n] == full["lse"][b, h, i]


# ---------------------------------------------------------------- dequantised inputs
def test_fp8_inputs_are_dequantised_with_scales(oracle_mod):
    x = torch.randn(1, 5, 2, 16, generator=torch.Generator().manual_seed(50))
    y = torch.randn(1, 9, 1, 16, generator=torch.Generator().manual_seed(51))
    z = torch.randn(1, 9, 1, 8, generator=torch.Generator().manual_seed(52))
    q8, sq = inputs.quantize_fp8(x)
    k8, sk = inputs.quantize_fp8(y)
    v8, sv = inputs.quantize_fp8(z)
    a = oracle_mod.sdpa(q8, k8, v8, scale=0.25, causal=True, descale=(sq, sk, sv))
    deq = lambda t, s: (t.to(torch.float64) * s).numpy()
    b = oracle_mod.sdpa(deq(q8, sq), deq(k8, sk), deq(v8, sv), scale=0.25, causal=True)
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], atol=1e-13)
    # quantisation error is within half an e4m3 ulp (3 fraction bits) of |x|/sigma
    rel = (deq(q8, sq) - x.double().numpy()) / sq
    assert np.abs(rel).max() <= 448.0 / 16 + 1e-9


def test_bf16_inputs_match_float64_widening(oracle_mod):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=33, kv_len=70)
    rows = np.array([[0, 0, 0], [0, 32, 31], [0, 17, 5]])
    a = oracle_mod.sdpa(q, k, v, scale=w.scale, causal=True, rows=rows)
    b = oracle_mod.sdpa(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=w.scale,
                        causal=True, rows=rows)
    assert np.array_equal(a["out"], b["out"])
