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
