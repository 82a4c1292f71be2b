"""The planner's load-balance figures (`range_iters_*` of sdpa_plan), checked
on the CPU against iteration counts recomputed here from the causal rule
itself: key j is visible to query i iff j <= i + kv_len - q_len, so a query
tile's K blocks are those up to its last row's last visible key, and every key
range of a workgroup runs ceil(blocks / ranges) iterations."""
import math

import numpy as np
import pytest

import attention_flash_sdpa_amd as sdpa
from attention_flash_sdpa_amd import inputs


def _expected(B, Sq, Sk, Hq, Hkv, causal, plan):
    """(max, min, sum) of the iterations per key range, from the definition:
    the workgroups of one query tile cover block_q rows of heads_per_group
    heads; their K blocks reach the last key any of those rows sees.  With
    the split across kv_splits workgroups, the blocks are cut into
    num_splits * kv_splits ranges of equal length, num_splits per
    workgroup; a workgroup whose first range starts past the last block runs
    none."""
    ks, kvs = plan.num_splits, plan.kv_splits
    iters = []
    for qt in range(math.ceil(Sq / plan.block_q)):
        last_row = min((qt + 1) * plan.block_q, Sq) - 1
        last_key = min(last_row + Sk - Sq, Sk - 1) if causal else Sk - 1
        blocks = math.ceil((last_key + 1) / plan.block_k) if last_key >= 0 else 0
        cnt = math.ceil(blocks / (ks * kvs))
        iters += [cnt if s * ks * cnt < blocks else 0 for s in range(kvs)]
    per_tile = plan.num_groups // len(iters)  # workgroups per (tile, split)
    assert per_tile * len(iters) == plan.num_groups
    assert per_tile == B * Hkv * math.ceil(Hq // Hkv / plan.heads_per_group)
    return max(iters), min(iters), sum(iters) * ks * per_tile


def _problem(B, Sq, Sk, Hq, Hkv, D, causal):
    return sdpa.make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=D,
                             in_dtype=sdpa.BF16, out_dtype=sdpa.BF16, causal=causal, scale=D ** -0.5)


def _plan(B, Sq, Sk, Hq, Hkv, D, causal):
    return sdpa.plan(_problem(B, Sq, Sk, Hq, Hkv, D, causal), num_cus=256)


def test_causal_gqa_workload_balance():
    """The causal GQA workload (512 queries over 1,024 keys, 32/8 heads): 256
    workgroups of two heads x 32 rows, two key ranges each.  Its 32-row tiles
    hold 9 to 16 K blocks, so ranges run 5 to 8 iterations, 6.5 on average:
    the busiest is 1.23x the mean."""
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    p = _plan(w.batch, w.q_len, w.kv_len, w.head_q, w.head_kv, w.d_qk, True)
    assert (p.num_groups, p.num_splits, p.block_q, p.block_k) == (256, 2, 32, 64)
    assert (p.range_iters_max, p.range_iters_min) == (8, 5)
    assert p.range_iters_sum == 256 * 2 * 6.5
    assert p.imbalance() == pytest.approx(8 / 6.5)


def test_full_attention_is_balanced():
    w = inputs.WORKLOADS["unaligned_full_bf16"]
    p = _plan(w.batch, w.q_len, w.kv_len, w.head_q, w.head_kv, w.d_qk, False)
    assert p.range_iters_max == p.range_iters_min == math.ceil(w.kv_len / 64)
    assert p.imbalance() == 1.0


@pytest.mark.parametrize("variant", [None, "narrow1", "narrow2", "occ2", "split4"])
def test_range_iterations_match_the_causal_rule(variant, prefill_variant):
    """Random shapes under every 16-bit form: the planner's figures equal the
    ones recomputed from the visibility rule."""
    prefill_variant(variant)
    g = np.random.default_rng(7 if variant is None else len(variant))
    for _ in range(40):
        Hkv = int(g.choice([1, 2, 8]))
        Hq = Hkv * int(g.choice([1, 2, 3, 4, 8]))
        B, Sq, Sk = int(g.integers(1, 4)), int(g.integers(1, 1500)), int(g.integers(1, 3000))
        causal = bool(g.integers(2))
        p = _plan(B, Sq, Sk, Hq, Hkv, 128, causal)
        mx, mn, total = _expected(B, Sq, Sk, Hq, Hkv, causal, p)
        assert (p.range_iters_max, p.range_iters_min, p.range_iters_sum) == (mx, mn, total), (B, Sq, Sk, Hq, Hkv,
                                                                                             causal, variant)
        assert p.imbalance() >= 1.0


def test_decode_plans_report_no_ranges():
    w = inputs.WORKLOADS["splitkv_decode_bf16"]
    p = sdpa.plan(_problem(w.batch, 1, w.kv_len, w.head_q, w.head_kv, w.d_qk, False), decode=True, num_cus=256)
    assert (p.range_iters_sum, p.range_iters_max, p.range_iters_min) == (0, 0, 0)
