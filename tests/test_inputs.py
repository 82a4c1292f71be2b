"""The seeded input generators shared by the GPU path and the oracle: same
seed, same tensors; pages hold exactly the dense keys; lengths cover the edge
values."""
import torch

from attention_flash_sdpa_amd import inputs


def test_make_qkv_is_deterministic_and_rotating_sets_differ():
    w = inputs.WORKLOADS["tiny_causal_bf16"]
    a = inputs.make_qkv(w)
    b = inputs.make_qkv(w)
    c = inputs.make_qkv(w, kv_set=1)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(a[0].view(torch.int16), c[0].view(torch.int16))        # Q from the base seed
    assert not torch.equal(a[1].view(torch.int16), c[1].view(torch.int16))    # K from the set's seed


def test_paginate_holds_every_key_once_and_fills_the_rest():
    g = torch.Generator().manual_seed(0)
    k = torch.randn(3, 70, 2, 8, generator=g).to(torch.bfloat16)
    v = torch.randn(3, 70, 2, 4, generator=g).to(torch.bfloat16)
    kp, vp, table = inputs.paginate(k, v, 16, seed=5, spare_pages=2)
    P = 5
    assert table.shape == (3, P) and table.dtype == torch.int32
    assert sorted(table.flatten().tolist()) == sorted(set(table.flatten().tolist()))   # no page used twice
    assert kp.shape == (3 * P + 2, 16, 2, 8) and vp.shape == (3 * P + 2, 16, 2, 4)
    for b in range(3):
        for j in range(70):
            p, r = table[b, j // 16], j % 16
            assert torch.equal(kp[p, r].view(torch.int16), k[b, j].view(torch.int16))
            assert torch.equal(vp[p, r].view(torch.int16), v[b, j].view(torch.int16))
        assert torch.isnan(kp[table[b, -1], 70 % 16:].float()).all()          # slots past the end
    spare = set(range(3 * P + 2)) - set(table.flatten().tolist())
    assert len(spare) == 2 and all(torch.isnan(kp[s].float()).all() for s in spare)
    assert torch.equal(inputs.paginate(k, v, 16, seed=5)[2], inputs.paginate(k, v, 16, seed=5)[2])


def test_length_mix_edges_and_range():
    lens = inputs.length_mix(7, 100, seed=3)
    assert lens.dtype == torch.int32 and lens[:3].tolist() == [0, 1, 100]
    assert ((lens >= 0) & (lens <= 100)).all()
    assert inputs.length_mix(2, 50, seed=1).tolist() == [0, 1]
    assert torch.equal(inputs.length_mix(7, 100, seed=3), lens)
