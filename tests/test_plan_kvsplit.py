"""The prefill split across workgroups (``plan.kv_splits``), on the CPU: when
the planner splits, the workspace it asks for, and a restatement of the
kernel's work decode showing that every K block a query tile sees is streamed
by exactly one key range and that every (batch, query row, query head, split)
partial row is written exactly once, empty splits included.

The restated decode follows the one-wave prefill kernel: block index ->
XCD-aware permutation -> (split, query tile, head group, KV head, batch);
the tile's n_blocks K blocks are cut into num_splits * kv_splits ranges of
ceil(n_blocks / (num_splits * kv_splits)) blocks; a workgroup whose first
range starts at or past n_blocks writes empty partials only."""
import ctypes
import math

import numpy as np
import pytest

import attention_flash_sdpa_amd as sdpa
from attention_flash_sdpa_amd import inputs


def _problem(B, Sq, Sk, Hq, Hkv, D, causal):
    return sdpa.make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=D,
                             in_dtype=sdpa.BF16, out_dtype=sdpa.BF16, causal=causal, scale=D ** -0.5)


def _remap_xcd(i, n):
    """Block i -> workgroup: blocks dealt round-robin to 8 XCDs get
    consecutive workgroup numbers on each XCD."""
    per, rem = n >> 3, n & 7
    x, j = i & 7, i >> 3
    return x * (per + 1) + j if x < rem else rem * (per + 1) + (x - rem) * per + j


def _tile_blocks(row0, row_end, Sq, Sk, bk, causal):
    """K blocks of a query tile: up to the last key its last row sees."""
    last_key = min(row_end - 1 + Sk - Sq, Sk - 1) if causal else Sk - 1
    return math.ceil((last_key + 1) / bk) if last_key >= 0 else 0


def _simulate(B, Sq, Sk, Hq, Hkv, causal, p):
    """(K blocks streamed for each (b, h, row), as a list of block ids;
    output rows written: array [B, Sq, Hq, kv_splits] of column halves
    written -- partials with a split, O and lse without)."""
    G = Hq // Hkv
    ks, nsp, hp = p.num_splits, max(p.kv_splits, 1), p.heads_per_group
    nws = p.waves_per_group // ks
    head_groups = math.ceil(G / hp)
    seen = {}
    writes = np.zeros((B, Sq, Hq, nsp), dtype=np.int64)
    assert sorted(_remap_xcd(i, p.num_groups) for i in range(p.num_groups)) == list(range(p.num_groups))
    for blk in range(p.num_groups):
        wg = _remap_xcd(blk, p.num_groups)
        ksp, wg = wg % nsp, wg // nsp
        qt, rest = wg % p.q_tiles, wg // p.q_tiles
        hg, rest = rest % head_groups, rest // head_groups
        g, b = rest % Hkv, rest // Hkv
        assert b < B
        if causal:
            qt = p.q_tiles - 1 - qt
        wg_row0 = qt * p.block_q
        wg_row_end = min(wg_row0 + p.block_q, Sq)
        n_blocks = _tile_blocks(wg_row0, wg_row_end, Sq, Sk, p.block_k, causal)
        nr = ks * nsp
        cnt = math.ceil(n_blocks / nr)
        empty = n_blocks == 0 or ksp * ks * cnt >= n_blocks
        for kr in range(ks):
            for wis in range(nws):
                hp_i, qp_i = wis % hp, wis // hp
                if hg * hp + hp_i >= G:
                    continue  # waves past the group's last head store nothing
                h = g * G + hg * hp + hp_i
                for l32 in range(32):
                    i = wg_row0 + 32 * qp_i + l32
                    if i >= Sq:
                        continue
                    if empty:
                        if kr == 0:
                            writes[b, i, h, ksp] += 2  # both halves of the row
                        continue
                    kb0 = (ksp * ks + kr) * cnt
                    blocks = [kb for kb in range(kb0, kb0 + cnt) if kb < n_blocks]
                    seen.setdefault((b, h, i), []).extend(blocks)
                    writes[b, i, h, ksp] += 1 if ks == 2 else 2  # one column half per range
    return seen, writes


SHAPES = [
    # B, Sq, Sk, Hq, Hkv, causal
    (1, 16, 8192, 32, 8, True),     # short chunk, long keys: the split's target
    (1, 16, 8192, 32, 8, False),
    (2, 5, 3000, 8, 2, True),
    (1, 64, 4096, 8, 8, True),      # two query tiles per head
    (1, 1, 2048, 4, 1, False),
    (3, 40, 999, 6, 3, True),       # ragged keys, odd group
    (1, 7, 5, 28, 4, True),         # fewer keys than a block, empty rows
    (1, 33, 700, 2, 1, False),
]


@pytest.mark.parametrize("variant", [None, "kvsplit", "kvsplit1"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_q{s[1]}_k{s[2]}_h{s[3]}x{s[4]}_{'c' if s[5] else 'f'}"
                                               for s in SHAPES])
def test_work_decode_covers_every_block_once(shape, variant, prefill_variant):
    B, Sq, Sk, Hq, Hkv, causal = shape
    prefill_variant(variant)
    p = sdpa.plan(_problem(B, Sq, Sk, Hq, Hkv, 128, causal), num_cus=256)
    if variant is not None:
        assert p.kv_splits >= 2 and p.num_splits == (2 if variant == "kvsplit" else 1) and p.kernel in (1, 3)
    seen, writes = _simulate(B, Sq, Sk, Hq, Hkv, causal, p)
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                qt = i // p.block_q
                row_end = min((qt + 1) * p.block_q, Sq)
                n_blocks = _tile_blocks(qt * p.block_q, row_end, Sq, Sk, p.block_k, causal)
                got = sorted(seen.get((b, h, i), []))
                assert got == list(range(n_blocks)), (b, h, i)
    # every partial row of every split written exactly once (both halves)
    assert (writes == 2).all()


def test_short_chunk_over_long_keys_splits_to_fill_the_gpu():
    """16 queries over 8,192 keys, 32/8 heads: 8 tiles of the four heads of a
    group, one key range each, split over 32 workgroups -> 256 workgroups of
    4 blocks, partials for 512 rows x 32 splits.  The two-range form would
    split 16 tiles of two heads 16 ways."""
    p = sdpa.plan(_problem(1, 16, 8192, 32, 8, 128, True), num_cus=256)
    assert (p.num_splits, p.kv_splits, p.num_groups, p.heads_per_group) == (1, 32, 256, 4)
    assert (p.range_iters_max, p.range_iters_min) == (4, 4)
    rows = 16 * 32
    po = rows * 32 * 128 * 4
    assert p.workspace_bytes == -(-po // 256) * 256 + rows * 32 * 2 * 4
    assert p.combine_groups == rows // 4


@pytest.mark.parametrize("Sk", [1000, 1200, 2048, 2049, 5000, 65536])
def test_auto_split_leaves_no_range_empty_on_full_attention(Sk):
    """Full attention: every split has work, ranges of four blocks or more,
    at least five iterations saved per range, at most one workgroup per CU."""
    p = sdpa.plan(_problem(1, 8, Sk, 16, 4, 64, False), num_cus=256)
    unsplit = math.ceil(p.kv_blocks / p.num_splits)
    if p.kv_splits > 1:
        assert p.range_iters_min == p.range_iters_max  # no empty workgroup
        assert p.range_iters_max >= 4  # no range shorter than four blocks
        assert unsplit - p.range_iters_max >= 5
        assert p.num_groups <= 256
    else:
        assert unsplit <= 9  # two ranges of half the blocks would save fewer than five


def test_workload_plans_do_not_split():
    """The measured workloads keep their one-kernel plans."""
    for name, w in inputs.WORKLOADS.items():
        if w.q_len == 1:
            continue
        codes = {"f16": sdpa.F16, "bf16": sdpa.BF16, "fp8_e4m3": sdpa.FP8_E4M3}
        pr = sdpa.make_problem(batch=w.batch, q_len=w.q_len, kv_len=w.kv_len, head_q=w.head_q, head_kv=w.head_kv,
                               d_qk=w.d_qk, d_v=w.d_v, in_dtype=codes[w.dtype], out_dtype=codes[w.out_dtype],
                               causal=w.causal, scale=1.0)
        p = sdpa.plan(pr, num_cus=256)
        assert p.kv_splits == 1 and p.workspace_bytes == 0, name


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv", [(3, 18, 5228, 32, 8), (1, 40, 9000, 12, 3), (2, 16, 20000, 40, 8)])
def test_auto_split_never_needs_a_second_round(B, Sq, Sk, Hq, Hkv):
    p = sdpa.plan(_problem(B, Sq, Sk, Hq, Hkv, 128, True), num_cus=256)
    assert p.kv_splits > 1 and p.num_groups <= 256


def test_workspace_query_matches_the_plan(prefill_variant):
    lib = sdpa.load()
    for variant in (None, "kvsplit", "kvsplit1", "narrow2"):
        prefill_variant(variant)
        for B, Sq, Sk, Hq, Hkv, causal in SHAPES:
            pr = _problem(B, Sq, Sk, Hq, Hkv, 64, causal)
            p = sdpa.plan(pr, num_cus=0)
            assert lib.sdpa_prefill_workspace_bytes(ctypes.byref(pr)) == p.workspace_bytes
            assert (p.workspace_bytes > 0) == (p.kv_splits > 1)
            if variant == "narrow2":
                assert p.kv_splits == 1


def test_cached_workspace_query_covers_cache_and_chunk(prefill_variant):
    """The cached prefill plans the whole sequence (cache + chunk): a 16-token
    chunk over 8,176 cached keys gets the workspace of a 16 x 8,192 prefill;
    nothing cached is the plain prefill's query."""
    lib = sdpa.load()
    chunk = _problem(1, 16, 16, 32, 8, 128, True)
    whole = sdpa.plan(_problem(1, 16, 8192, 32, 8, 128, True), num_cus=0)
    assert whole.kv_splits > 1
    assert lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(chunk), 8176) == whole.workspace_bytes
    assert lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(chunk), 0) == \
        lib.sdpa_prefill_workspace_bytes(ctypes.byref(chunk)) == 0
    assert lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(chunk), -1) == 0
    prefill_variant("narrow2")
    assert lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(chunk), 8176) == 0
