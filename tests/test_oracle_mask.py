"""Pins of the mask conversion oracle (oracle/mask.py): IEEE encodings of 0
and -inf in both 16-bit types, torch's own casts, and what adding the result
to scores does."""
import numpy as np
import torch

from oracle import mask as om


def test_encodings_are_ieee_zero_and_minus_infinity():
    m = np.array([0, 1, 2, 255, 0], dtype=np.uint8)
    f = om.mask_convert(m, "f16")
    assert f.view(np.uint16).tolist() == [0xFC00, 0, 0, 0, 0xFC00]       # binary16 -inf is 0xfc00
    b = om.mask_convert(m, "bf16")
    assert b.tolist() == [0xFF80, 0, 0, 0, 0xFF80]                          # bfloat16 -inf is 0xff80


def test_matches_torch_casts_of_zero_and_minus_infinity():
    g = torch.Generator().manual_seed(0)
    m = (torch.rand(3, 5, 7, generator=g) < 0.5).to(torch.uint8) * torch.randint(1, 256, (3, 5, 7), generator=g,
                                                                                 dtype=torch.uint8)
    want = torch.where(m != 0, 0.0, float("-inf"))
    b = om.mask_convert(m.numpy(), "bf16")
    assert np.array_equal(b, want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    f = om.mask_convert(m.numpy(), "f16")
    assert np.array_equal(f.view(np.uint16), want.to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    assert f.shape == (3, 5, 7)


def test_adding_the_mask_removes_exactly_the_blocked_keys_from_a_softmax():
    g = torch.Generator().manual_seed(1)
    s = torch.randn(4, 9, generator=g, dtype=torch.float64)
    m = (torch.rand(4, 9, generator=g) < 0.6).to(torch.uint8)
    m[:, 0] = 1
    add = torch.from_numpy(om.mask_convert(m.numpy(), "f16").astype(np.float64))
    p = torch.softmax(s + add, dim=1)
    keep = m.bool()
    want = torch.where(keep, torch.exp(s), 0.0)
    want = want / want.sum(1, keepdim=True)
    assert torch.allclose(p, want, atol=1e-15) and (p[~keep] == 0).all()


def _qkv(B, Sq, Sk, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Sq, Hq, D, generator=g).to(torch.bfloat16),
            torch.randn(B, Sk, Hkv, D, generator=g).to(torch.bfloat16),
            torch.randn(B, Sk, Hkv, D, generator=g).to(torch.bfloat16))


def test_zero_mask_is_the_plain_prefill():
    import oracle

    q, k, v = _qkv(2, 19, 23, 4, 2, 16, 0)
    for causal in (False, True):
        got = om.prefill_masked(q, k, v, torch.zeros(1, 1, 19, 23), scale=0.3, causal=causal)
        want = oracle.sdpa(q, k, v, scale=0.3, causal=causal)
        assert np.abs(got["out"] - want["out"]).max() < 1e-12
        assert np.abs(got["lse"] - want["lse"]).max() < 1e-12


def test_minus_infinity_entries_remove_exactly_those_keys():
    """A 0 / -inf mask from mask_convert equals the plain definition over the
    kept keys (row by row), and a causal 0 / -inf mask equals causal=True."""
    import oracle

    q, k, v = _qkv(1, 6, 20, 2, 1, 16, 1)
    g = torch.Generator().manual_seed(2)
    keep = torch.rand(1, 1, 6, 20, generator=g) < 0.6
    keep[..., 0] = True
    add = torch.from_numpy(om.mask_convert(keep.numpy().astype(np.uint8), "f16").astype(np.float32))
    got = om.prefill_masked(q, k, v, add, scale=0.25, causal=False)
    for i in range(6):
        idx = torch.nonzero(keep[0, 0, i])[:, 0]
        want = oracle.sdpa(q[:, i:i + 1], k[:, idx], v[:, idx], scale=0.25, causal=False)
        assert np.abs(got["out"][:, i] - want["out"][:, 0]).max() < 1e-12
    i = torch.arange(6)[:, None]
    j = torch.arange(20)[None, :]
    cmask = torch.where(j <= i + 14, 0.0, float("-inf"))[None, None]
    a = om.prefill_masked(q, k, v, cmask, scale=0.25, causal=False)
    b = oracle.sdpa(q, k, v, scale=0.25, causal=True)
    assert np.abs(a["out"] - b["out"]).max() < 1e-12


def test_row_constant_shifts_leave_o_and_move_lse():
    q, k, v = _qkv(1, 5, 9, 2, 2, 8, 3)
    g = torch.Generator().manual_seed(4)
    base = torch.randn(1, 2, 5, 9, generator=g, dtype=torch.float64)
    c = torch.randn(1, 2, 5, 1, generator=g, dtype=torch.float64)
    a = om.prefill_masked(q, k, v, base, scale=0.5, causal=False)
    b = om.prefill_masked(q, k, v, base + c, scale=0.5, causal=False)
    assert np.abs(a["out"] - b["out"]).max() < 1e-12
    assert np.abs((b["lse"] - a["lse"]) - c[0, :, :, 0].numpy()[None]).max() < 1e-12


def test_broadcast_equals_the_materialised_mask():
    q, k, v = _qkv(2, 7, 11, 4, 2, 8, 5)
    g = torch.Generator().manual_seed(6)
    m = torch.randn(1, 4, 7, 11, generator=g)
    a = om.prefill_masked(q, k, v, m, scale=0.4, causal=True)
    b = om.prefill_masked(q, k, v, m.expand(2, 4, 7, 11).contiguous(), scale=0.4, causal=True)
    assert np.array_equal(a["out"], b["out"])
    m1 = torch.randn(2, 1, 7, 11, generator=g)
    a = om.prefill_masked(q, k, v, m1, scale=0.4, causal=False)
    b = om.prefill_masked(q, k, v, m1.expand(2, 4, 7, 11).contiguous(), scale=0.4, causal=False)
    assert np.array_equal(a["out"], b["out"])
