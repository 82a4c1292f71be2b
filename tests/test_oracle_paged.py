"""Pins of the paged / variable-length decode oracle (oracle/paged.py): the
page-table gather must reduce to the plain definition on contiguous keys."""
import numpy as np
import pytest
import torch

import oracle
from oracle import paged


def _contiguous(B=3, Sk=200, Hq=8, Hkv=2, D=64, seed=0, dt=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    return q, k, v


def _paginate(k, page_size, pages_per_seq, perm_seed=None):
    """Contiguous [B, Sk, H, D] -> pool [B*pages_per_seq, page_size, H, D] and
    its page table; with perm_seed the physical pages are shuffled."""
    B, Sk, H, D = k.shape
    pad = pages_per_seq * page_size - Sk
    kp = torch.cat([k, torch.zeros(B, pad, H, D, dtype=k.dtype)], dim=1)
    pool = kp.reshape(B * pages_per_seq, page_size, H, D)
    table = np.arange(B * pages_per_seq, dtype=np.int32).reshape(B, pages_per_seq)
    if perm_seed is not None:
        perm = np.random.default_rng(perm_seed).permutation(B * pages_per_seq)
        inv = np.argsort(perm)
        pool = pool[torch.as_tensor(perm)]          # physical page i holds logical page perm[i]
        table = inv[table].astype(np.int32)          # logical page -> its new physical slot
    return pool, table


def test_identity_table_equals_contiguous_definition():
    q, k, v = _contiguous()
    kp, table = _paginate(k, 32, 7)
    vp, _ = _paginate(v, 32, 7)
    want = oracle.sdpa(q[:, None], k, v, scale=0.125, causal=False)
    got = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=[200] * 3,
                             scale=0.125)
    assert np.array_equal(got["out"], want["out"][:, 0])
    assert np.array_equal(got["lse"], want["lse"][:, :, 0])


def test_without_lengths_every_sequence_is_full():
    """No seq_lens: a paged sequence holds its whole table row (not one page),
    or kv_len keys when kv_len is given."""
    q, k, v = _contiguous(Sk=192)
    kp, table = _paginate(k, 32, 6, perm_seed=2)
    vp, _ = _paginate(v, 32, 6, perm_seed=2)
    want = oracle.sdpa(q[:, None], k, v, scale=0.125, causal=False)
    got = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=None, scale=0.125)
    assert np.array_equal(got["out"], want["out"][:, 0])
    short = oracle.sdpa(q[:, None], k[:, :100], v[:, :100], scale=0.125, causal=False)
    got = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=None, scale=0.125, kv_len=100)
    assert np.array_equal(got["out"], short["out"][:, 0])
    got = paged.decode_paged(q, k, v, page_table=None, page_size=0, seq_lens=None, scale=0.125)
    assert np.array_equal(got["out"], want["out"][:, 0])


def test_shuffled_physical_pages_do_not_change_the_result():
    q, k, v = _contiguous(seed=1)
    kp, table = _paginate(k, 64, 4, perm_seed=5)
    vp, _ = _paginate(v, 64, 4, perm_seed=5)
    want = oracle.sdpa(q[:, None], k, v, scale=0.2, causal=False)["out"][:, 0]
    got = paged.decode_paged(q, kp, vp, page_table=table, page_size=64, seq_lens=[200] * 3, scale=0.2)["out"]
    assert np.array_equal(got, want)


def test_variable_lengths_equal_truncated_definition():
    q, k, v = _contiguous(seed=2)
    lens = [200, 1, 77]
    kp, table = _paginate(k, 32, 7, perm_seed=9)
    vp, _ = _paginate(v, 32, 7, perm_seed=9)
    got = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=lens, scale=0.125)
    got_c = paged.decode_paged(q, k, v, page_table=None, page_size=0, seq_lens=lens, scale=0.125)
    for b, n in enumerate(lens):
        want = oracle.sdpa(q[b:b + 1, None], k[b:b + 1, :n], v[b:b + 1, :n], scale=0.125, causal=False)
        assert np.array_equal(got["out"][b], want["out"][0, 0])
        assert np.array_equal(got_c["out"][b], want["out"][0, 0])
    # one key: the output is that key's value row (per KV head group)
    G = q.shape[1] // k.shape[2]
    for h in range(q.shape[1]):
        assert np.allclose(got["out"][1, h], v[1, 0, h // G].double().numpy(), rtol=0, atol=0)


def test_empty_sequence_gives_zero_and_minus_inf():
    q, k, v = _contiguous(B=2, seed=3)
    kp, table = _paginate(k, 32, 7)
    vp, _ = _paginate(v, 32, 7)
    r = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=[0, 5], scale=0.125)
    assert (r["out"][0] == 0).all() and np.isneginf(r["lse"][0]).all()
    assert np.isfinite(r["lse"][1]).all()


def test_a_wrong_table_entry_is_noticed():
    """The pins above would miss a gather that ignores the table; a table that
    points one logical page at another page must change the result."""
    q, k, v = _contiguous(seed=4)
    kp, table = _paginate(k, 32, 7)
    vp, _ = _paginate(v, 32, 7)
    bad = table.copy()
    bad[0, 2] = table[1, 2]
    good = paged.decode_paged(q, kp, vp, page_table=table, page_size=32, seq_lens=[200] * 3, scale=0.125)["out"]
    wrong = paged.decode_paged(q, kp, vp, page_table=bad, page_size=32, seq_lens=[200] * 3, scale=0.125)["out"]
    assert not np.allclose(good[0], wrong[0]) and np.array_equal(good[1:], wrong[1:])
