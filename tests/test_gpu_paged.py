"""GPU parity of the variable-length / paged decode (``sdpa_decode_paged_fwd``)
against the fp64 oracle ``oracle.paged.decode_paged``.

Pools come from ``inputs.paginate``: physical pages in a seeded random order,
spare pages and the slots past each sequence's end filled with NaN, so a read
of any slot a sequence does not own turns up as a NaN in its output.  Bar as
for the dense decode: no NaN, max |gpu - oracle| <= 2e-2 on O, the lse bound
of the dense tests, and -inf / 0 exactly for an empty sequence.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_flash_sdpa_amd as sdpa
from attention_flash_sdpa_amd import inputs

pytestmark = pytest.mark.gpu

TOL16 = 2e-2


def _lse_tol(dtype):
    """lse from fp32 row sums of the fp32 probabilities: the sequential sum of
    n terms is within n * 2^-24 relative, 1e-3 covers rows of 16K keys."""
    return 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sdpa.load()
    return torch.device("cuda:0")


def _draw(B, Sk, Hq, Hkv, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    return q, k, v


def _run(dev, q, kc, vc, *, table, lens, kv_len, splits=0):
    B, Hq, _ = q.shape
    out = torch.full((B, Hq, vc.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), page_table=None if table is None else table.to(dev),
                      seq_lens=None if lens is None else lens.to(dev), kv_len=kv_len, out=out, lse=lse,
                      num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


def _check(out, lse, ref, dtype):
    got = out.double().cpu().numpy()
    nan = int(np.isnan(got).sum())
    err = np.abs(got - ref["out"])
    worst = float(err.max()) if err.size else 0.0
    _say(f"  out: nan={nan} max_abs={worst:.3e}")
    assert nan == 0 and worst <= TOL16, (nan, worst)
    gl = lse.double().cpu().numpy()
    want = ref["lse"]
    assert np.array_equal(np.isneginf(gl), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.abs(gl[fin] - want[fin]).max(initial=0) <= _lse_tol(dtype)


PAGED = [
    # B, kv_len, Hq, Hkv, D, dtype, page_size, splits, lengths ("mix" or "full")
    (4, 1000, 8, 2, 128, torch.bfloat16, 64, 0, "mix"),
    (6, 777, 16, 4, 64, torch.float16, 32, 0, "mix"),
    (2, 2048, 32, 8, 128, torch.bfloat16, 128, 5, "full"),
    (5, 300, 4, 1, 128, torch.bfloat16, 96, 0, "mix"),     # page size not a power of two
    (3, 450, 12, 3, 64, torch.bfloat16, 32, 40, "mix"),    # many splits, most of them empty
    (1, 8192, 4, 1, 64, torch.bfloat16, 32, 1, "full"),    # 256 pages in one split: table reloads
    (3, 5000, 6, 2, 128, torch.float16, 32, 2, "mix"),     # 79 pages per split: table reloads, lengths 0, 1, full
    (4, 3000, 16, 1, 128, torch.bfloat16, 256, 0, "mix"),  # 16 query heads per KV head, 256-key pages
    (2, 640, 12, 12, 64, torch.float16, 64, 3, "full"),    # no grouping (MHA)
    (4, 1000, 8, 2, 128, torch.bfloat16, 16, 0, "mix"),    # 16-key pages: two pages per block
    (3, 777, 16, 4, 64, torch.float16, 8, 0, "mix"),       # 8-key pages: four pages per block
    (3, 5000, 6, 2, 128, torch.bfloat16, 8, 2, "mix"),     # 8-key pages, 316 pages per split: table reloads
    (3, 1200, 64, 2, 128, torch.bfloat16, 64, 0, "mix"),   # 32 query heads per KV head (two 16-head tiles)
]


@pytest.mark.parametrize("case", PAGED, ids=[f"B{c[0]}_k{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_p{c[6]}_s{c[7]}_{c[8]}"
                                             for c in PAGED])
def test_paged_decode(dev, case):
    from oracle import paged as op

    B, Sk, Hq, Hkv, D, dt, ps, splits, mode = case
    seed = Sk + 31 * Hq + ps
    _say(f"paged decode B={B} kv_len={Sk} Hq={Hq} Hkv={Hkv} D={D} {dt} page={ps} splits={splits} {mode}")
    q, k, v = _draw(B, Sk, Hq, Hkv, D, dt, seed)
    kp, vp, table = inputs.paginate(k, v, ps, seed=seed + 1, spare_pages=3)
    lens = inputs.length_mix(B, Sk, seed=seed + 2) if mode == "mix" else None
    out, lse = _run(dev, q, kp, vp, table=table, lens=lens, kv_len=Sk, splits=splits)
    ref = op.decode_paged(q, kp, vp, page_table=table, page_size=ps, seq_lens=None if lens is None else lens.tolist(),
                          scale=1 / math.sqrt(D), kv_len=Sk)
    _check(out, lse, ref, dt)


VARLEN = [
    (5, 500, 8, 2, 128, torch.float16, 0),
    (4, 129, 16, 16, 64, torch.bfloat16, 3),
]


@pytest.mark.parametrize("case", VARLEN, ids=[f"B{c[0]}_k{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_s{c[6]}" for c in VARLEN])
def test_dense_variable_length_decode(dev, case):
    from oracle import paged as op

    B, Sk, Hq, Hkv, D, dt, splits = case
    _say(f"variable-length dense decode B={B} kv_len={Sk} Hq={Hq} Hkv={Hkv} D={D} {dt} splits={splits}")
    q, k, v = _draw(B, Sk, Hq, Hkv, D, dt, Sk + 7)
    lens = inputs.length_mix(B, Sk, seed=Sk + 8)
    out, lse = _run(dev, q, k, v, table=None, lens=lens, kv_len=Sk, splits=splits)
    ref = op.decode_paged(q, k, v, page_table=None, page_size=0, seq_lens=lens.tolist(), scale=1 / math.sqrt(D))
    _check(out, lse, ref, dt)


def test_identity_table_matches_dense_decode_bitwise(dev):
    """With pages in logical order and every sequence full, the paged call runs
    the same blocks and splits as the dense decode: identical bits."""
    B, Sk, Hq, Hkv, D, ps = 3, 1024, 16, 4, 128, 64
    _say(f"identity table vs dense decode B={B} kv_len={Sk} page={ps}")
    q, k, v = _draw(B, Sk, Hq, Hkv, D, torch.bfloat16, 99)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    dense = sdpa.decode(qd, kd, vd)
    table = torch.arange(B * (Sk // ps), dtype=torch.int32).reshape(B, -1).to(dev)
    pool_k = kd.reshape(B * (Sk // ps), ps, Hkv, D)
    pool_v = vd.reshape(B * (Sk // ps), ps, Hkv, D)
    paged = sdpa.decode_paged(qd, pool_k, pool_v, page_table=table)
    full = torch.full((B,), Sk, dtype=torch.int32, device=dev)
    varlen = sdpa.decode_paged(qd, kd, vd, seq_lens=full)
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), paged.view(torch.int16))
    assert torch.equal(dense.view(torch.int16), varlen.view(torch.int16))


def test_paged_decode_workload_full_size(dev):
    """The bf16 decode workload (16 sequences, 32 query / 8 KV heads, 8192
    keys, head dim 128) in 64-key pages, shuffled, with mixed lengths."""
    from oracle import paged as op

    w = inputs.WORKLOADS["splitkv_decode_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    q = q.reshape(w.batch, w.head_q, w.d_qk)
    kp, vp, table = inputs.paginate(k, v, 64, seed=w.seed + 1, spare_pages=8)
    del k, v
    lens = inputs.length_mix(w.batch, w.kv_len, seed=w.seed + 2)
    _say(f"paged decode workload lens={lens.tolist()}")
    out, lse = _run(dev, q, kp, vp, table=table, lens=lens, kv_len=w.kv_len)
    ref = op.decode_paged(q, kp, vp, page_table=table, page_size=64, seq_lens=lens.tolist(), scale=w.scale)
    _check(out, lse, ref, q.dtype)


def test_out_of_range_table_entry_poisons_only_its_sequence(dev):
    """Entries outside [0, num_pages) are never dereferenced (the kernel
    checks each one before use); they turn that sequence's rows into NaN and
    leave the others exact."""
    from oracle import paged as op

    B, Sk, Hq, Hkv, D, ps = 4, 256, 8, 2, 64, 32
    q, k, v = _draw(B, Sk, Hq, Hkv, D, torch.bfloat16, 5)
    kp, vp, table = inputs.paginate(k, v, ps, seed=6, fill=0.0)
    bad = table.clone()
    bad[1, 3] = kp.shape[0] + 3
    bad[2, 0] = -1
    _say("paged decode with out-of-range table entries in sequences 1 and 2")
    out, lse = _run(dev, q, kp, vp, table=bad, lens=None, kv_len=Sk)
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(ls[1]).all() and np.isnan(ls[2]).all()
    ref = op.decode_paged(q, kp, vp, page_table=table, page_size=ps, seq_lens=None, scale=1 / math.sqrt(D),
                          kv_len=Sk)
    keep = [0, 3]
    assert np.abs(o[keep] - ref["out"][keep]).max() <= TOL16
    assert np.abs(ls[keep] - ref["lse"][keep]).max() <= _lse_tol(torch.bfloat16)


def test_paged_decode_empty_batch_and_zero_lengths(dev):
    q = torch.randn(3, 8, 128).to(torch.bfloat16).to(dev)
    pool = torch.zeros(4, 64, 2, 128, dtype=torch.bfloat16, device=dev)
    table = torch.zeros(3, 2, dtype=torch.int32, device=dev)
    lens = torch.zeros(3, dtype=torch.int32, device=dev)
    out = torch.full((3, 8, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(3, 8, device=dev)
    sdpa.decode_paged(q, pool, pool, page_table=table, seq_lens=lens, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    empty = sdpa.decode_paged(q[:0], pool, pool, page_table=table[:0])
    assert empty.shape == (0, 8, 128)


def test_dense_kv_len_beyond_the_cache_is_rejected(dev):
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(2, 64, 2, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        sdpa.decode_paged(q, k, k, kv_len=65)


@pytest.mark.parametrize("ps", [8, 16, 64])
def test_table_entries_past_the_sequence_end_are_ignored(dev, ps):
    """Entries of a table row past a sequence's last page may hold anything
    (here out-of-range values): they are never used and poison nothing."""
    from oracle import paged as op

    B, Sk, Hq, Hkv, D = 4, 300, 8, 2, 64
    q, k, v = _draw(B, Sk, Hq, Hkv, D, torch.bfloat16, 21 + ps)
    kp, vp, table = inputs.paginate(k, v, ps, seed=22, spare_pages=1)
    lens = torch.tensor([0, 1, 77, 300], dtype=torch.int32)
    garbage = table.clone()
    for b in range(B):
        garbage[b, -(-int(lens[b]) // ps):] = -7 - b
    _say(f"garbage past the sequence ends, page {ps}")
    out, lse = _run(dev, q, kp, vp, table=garbage, lens=lens, kv_len=Sk)
    ref = op.decode_paged(q, kp, vp, page_table=table, page_size=ps, seq_lens=lens.tolist(), scale=1 / math.sqrt(D))
    _check(out, lse, ref, torch.bfloat16)


@pytest.mark.parametrize("ps", [8, 16])
def test_small_page_out_of_range_entry_poisons_its_sequence(dev, ps):
    from oracle import paged as op

    B, Sk, Hq, Hkv, D = 3, 200, 4, 1, 128
    q, k, v = _draw(B, Sk, Hq, Hkv, D, torch.bfloat16, 31 + ps)
    kp, vp, table = inputs.paginate(k, v, ps, seed=32, fill=0.0)
    bad = table.clone()
    bad[1, 5] = kp.shape[0]
    _say(f"out-of-range entry with {ps}-key pages")
    out, lse = _run(dev, q, kp, vp, table=bad, lens=None, kv_len=Sk)
    o = out.double().cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(lse[1].cpu().numpy()).all()
    ref = op.decode_paged(q, kp, vp, page_table=table, page_size=ps, seq_lens=None, scale=1 / math.sqrt(D),
                          kv_len=Sk)
    assert np.abs(o[[0, 2]] - ref["out"][[0, 2]]).max() <= TOL16
