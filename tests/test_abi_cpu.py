"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
symbol include/sdpa.h declares, validates arguments, and its planner reproduces
the loop counts printed on the pages and plans the workloads sensibly."""
import json
import os
import re

import pytest

import attention_flash_sdpa_amd as sdpa
from attention_flash_sdpa_amd import binding, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "sdpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sdpa.load()
    declared = _header_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(binding.EXPORTS)
    assert lib.sdpa_abi_version() == 3


def test_status_strings():
    lib = sdpa.load()
    for code in range(8):
        assert lib.sdpa_status_string(code).startswith(b"SDPA_")
    assert b"unknown" in lib.sdpa_status_string(99)


def test_page_loop_counts_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "sagev1_loop_counts.json")))
    p, t, e = g["problem"], g["tile"], g["expected"]
    c = sdpa.loop_counts(q_len=p["q_len"], kv_len=p["kv_len"], d_qk=p["d_qk"], d_v=p["d_v"], block_q=t["block_q"],
                         block_k=t["block_k"], block_d=t["block_d"], block_v=t["block_v"], causal=p["causal"])
    assert c.q_blocks == e["q_blocks"]
    assert c.k_blocks == e["k_blocks"]
    assert c.d_loops == e["d_loops_per_k_block"]
    assert c.vv_loops == e["vv_loops_per_k_block"]
    assert c.blocks_visited // c.q_blocks == e["per_q_block"]["k_blocks"]
    assert c.qk_tiles // c.q_blocks == e["per_q_block"]["qk_tiles"]
    assert c.pv_tiles // c.q_blocks == e["per_q_block"]["pv_tiles"]
    assert c.softmax_tiles // c.q_blocks == e["per_q_block"]["softmax_tiles"]
    assert c.qk_tiles == e["per_head"]["qk_tiles"]
    assert c.pv_tiles == e["per_head"]["pv_tiles"]
    assert c.softmax_tiles == e["per_head"]["softmax_tiles"]
    assert c.blocks_masked == 0


def _brute_blocks(q_len, kv_len, bq, bk, causal):
    """Blocks visited / masked by brute force over every (row, key) pair."""
    visited = masked = 0
    for r0 in range(0, q_len, bq):
        rows = range(r0, min(r0 + bq, q_len))
        for kb in range(0, kv_len, bk):
            keys = range(kb, min(kb + bk, kv_len))
            vis = [[(not causal) or (j <= i + kv_len - q_len) for j in keys] for i in rows]
            n_vis = sum(map(sum, vis))
            if n_vis:
                visited += 1
                if n_vis != len(rows) * bk:
                    masked += 1
            elif causal:
                # a causal row block sees a prefix of keys; nothing visible
                # in this block means nothing visible in later blocks either
                break
    return visited, masked


@pytest.mark.parametrize("q_len,kv_len,causal", [(512, 1024, True), (1001, 1023, False), (7, 5, True),
                                                   (5, 7, True), (33, 64, True), (64, 64, True), (1, 8192, False),
                                                   (130, 2, True), (3, 0, False), (0, 5, True)])
@pytest.mark.parametrize("bq,bk", [(32, 64), (128, 64), (256, 64)])
def test_loop_counts_match_brute_force(q_len, kv_len, causal, bq, bk):
    c = sdpa.loop_counts(q_len=q_len, kv_len=kv_len, d_qk=128, d_v=128, block_q=bq, block_k=bk, block_d=16,
                         block_v=32, causal=causal)
    v, m = _brute_blocks(q_len, kv_len, bq, bk, causal)
    assert (c.blocks_visited, c.blocks_masked) == (v, m)


def _problem(w: inputs.Workload, **over):
    code = {"f16": sdpa.F16, "bf16": sdpa.BF16, "fp8_e4m3": sdpa.FP8_E4M3}
    d = dict(batch=w.batch, q_len=w.q_len, kv_len=w.kv_len, head_q=w.head_q, head_kv=w.head_kv, d_qk=w.d_qk,
             d_v=w.d_v, in_dtype=code[w.dtype], out_dtype=code[w.out_dtype], causal=w.causal, scale=w.scale)
    d.update(over)
    return sdpa.make_problem(**d)


def test_plans_for_workloads():
    W = inputs.WORKLOADS
    p = sdpa.plan(_problem(W["gqa_causal_prefill_bf16"]))
    # 4 heads x 1 tile would give 128 workgroups (< 256 CUs): the key range of
    # each workgroup is split in two, 2 heads x 2 ranges
    assert (p.rows_per_wave, p.heads_per_group, p.block_q, p.block_k, p.q_tiles, p.kv_blocks) == (32, 2, 32, 64, 16, 16)
    assert p.num_splits == 2 and p.num_groups == 8 * 2 * 16 and p.workspace_bytes == 0 and p.lds_bytes == 131072
    assert sdpa.plan(_problem(W["gqa_causal_prefill_bf16"]), num_cus=128).num_splits == 1
    p = sdpa.plan(_problem(W["unaligned_full_bf16"]))
    assert (p.rows_per_wave, p.heads_per_group, p.qtiles_per_group, p.q_tiles, p.block_k) == (32, 1, 4, 8, 64)
    assert p.num_groups == 2 * 4 * 7 * 8 and p.num_splits == 1
    assert p.kernel == 15   # 448 workgroups > 256 CUs: the two-waves-per-SIMD form
    assert sdpa.plan(_problem(W["gqa_causal_prefill_bf16"])).kernel == 3
    p = sdpa.plan(_problem(W["tiny_causal_bf16"]))
    assert (p.heads_per_group, p.q_tiles, p.num_groups) == (4, 1, 2 * 4 * 2)
    d = sdpa.plan(_problem(W["splitkv_decode_bf16"]), decode=True, num_cus=256)
    # 128 KiB of LDS per workgroup: one per CU, so one round of 256 workgroups
    assert (d.num_splits, d.blocks_per_split, d.block_k) == (8, 32, 32)
    assert d.num_groups * d.waves_per_group == 16 * 8 * 8 and d.num_groups == 256
    assert d.combine_groups == 16 * 32 // 4   # four (batch, head) rows per workgroup
    assert d.workspace_bytes == 16 * 32 * 8 * 128 * 4 + 16 * 32 * 8 * 2 * 4
    # d = 64 blocks take 64 KiB: two workgroups per CU
    import dataclasses
    d64 = sdpa.plan(_problem(dataclasses.replace(W["splitkv_decode_bf16"], d_qk=64, d_v=64)), decode=True, num_cus=256)
    assert d64.num_splits == 16 and d64.num_groups == 512


def test_decode_large_groups_take_one_wave_per_16_heads():
    """More than 16 query heads per KV head: one wave per (KV head, tile of up
    to 16 query heads), four such tasks per workgroup."""
    import dataclasses

    w = dataclasses.replace(inputs.WORKLOADS["splitkv_decode_bf16"], head_q=64, head_kv=2)   # G = 32
    d = sdpa.plan(_problem(w), decode=True, num_cus=256)
    tasks = 16 * 2 * 2   # batch x KV heads x tiles
    assert d.num_groups == 16 * d.num_splits * ((2 * 2 + 3) // 4)
    assert d.num_splits == min(-(-256 * 4 // tasks), 8192 // 32 // 2)
    w20 = dataclasses.replace(w, head_q=20, head_kv=1, batch=1)   # G = 20: tiles of 16 and 4
    d20 = sdpa.plan(_problem(w20), decode=True, num_cus=256)
    assert d20.num_groups == d20.num_splits * 1   # 2 tasks fit one workgroup
    assert d20.workspace_bytes == 1 * 20 * d20.num_splits * (128 * 4 + 8)


def test_prefill_variant_override(prefill_variant):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    prefill_variant("narrow1")
    p1 = sdpa.plan(_problem(w))
    assert (p1.num_splits, p1.heads_per_group, p1.num_groups, p1.lds_bytes) == (1, 4, 128, 65536)
    prefill_variant("narrow2")
    p2 = sdpa.plan(_problem(inputs.WORKLOADS["unaligned_full_bf16"]))
    assert (p2.num_splits, p2.heads_per_group, p2.qtiles_per_group, p2.num_groups) == (2, 1, 2, 2 * 4 * 7 * 16)
    prefill_variant("split4")
    p4 = sdpa.plan(_problem(w))
    assert (p4.kernel, p4.num_splits, p4.waves_per_group, p4.block_k, p4.kv_blocks) == (27, 4, 8, 32, 32)
    assert (p4.heads_per_group, p4.qtiles_per_group, p4.num_groups, p4.lds_bytes) == (2, 1, 8 * 2 * 16, 131072)
    with pytest.raises(sdpa.SdpaError, match="UNSUPPORTED"):
        prefill_variant("wide")   # unknown names change nothing
    assert sdpa.plan(_problem(w)).num_splits == 4
    prefill_variant(None)
    assert sdpa.plan(_problem(w)).rows_per_wave == 32 and sdpa.plan(_problem(w)).num_splits == 2


def test_descale_must_be_one_for_16bit_inputs():
    """Dequantisation factors belong to fp8 inputs; with fp16/bf16 inputs any
    factor other than 1 is rejected by the planner, so every entry point
    (prefill, cached, masked, decode, paged) refuses it before a launch."""
    for name in ("gqa_causal_prefill_bf16", "single_head_f16_128"):
        w = inputs.WORKLOADS[name]
        for ds in ((2.0, 1.0, 1.0), (1.0, 0.5, 1.0), (1.0, 1.0, 3.0)):
            pr = sdpa.make_problem(batch=w.batch, q_len=w.q_len, kv_len=w.kv_len, head_q=w.head_q,
                                   head_kv=w.head_kv, d_qk=w.d_qk, d_v=w.d_v,
                                   in_dtype=sdpa.BF16 if w.dtype == "bf16" else sdpa.F16,
                                   out_dtype=sdpa.BF16 if w.dtype == "bf16" else sdpa.F16, causal=w.causal,
                                   scale=w.scale, descale=ds)
            for dec in (False, True):
                if dec:
                    pr.q_len = 1
                with pytest.raises(sdpa.SdpaError, match="BAD_SCALE"):
                    sdpa.plan(pr, decode=dec)
    w = inputs.WORKLOADS["mla_fp8_causal_prefill"]
    pr = sdpa.make_problem(batch=1, q_len=w.q_len, kv_len=w.kv_len, head_q=w.head_q, head_kv=w.head_kv,
                           d_qk=w.d_qk, d_v=w.d_v, in_dtype=sdpa.FP8_E4M3, out_dtype=sdpa.BF16, causal=True,
                           scale=w.scale, descale=(0.01, 0.02, 0.03))
    sdpa.plan(pr)   # fp8: any finite factor >= 0


def test_decode_split_choices():
    w = inputs.WORKLOADS["splitkv_decode_bf16"]
    for kv_len, cus in ((1, 256), (31, 256), (64, 256), (100000, 256), (8192, 80)):
        d = sdpa.plan(_problem(w, kv_len=kv_len), decode=True, num_cus=cus)
        blocks = -(-kv_len // 32)
        assert d.num_splits >= 1 and d.blocks_per_split >= 1
        assert d.num_splits * d.blocks_per_split >= blocks                 # covers every key
        assert (d.num_splits - 1) * d.blocks_per_split < blocks            # no empty split
    forced = sdpa.plan(_problem(w, kv_len=100), decode=True, num_splits=9)
    assert forced.num_splits == 9 and forced.blocks_per_split == 1      # 4 blocks: 5 empty splits allowed


@pytest.mark.parametrize("over,decode,code", [
    (dict(head_q=30), False, 2), (dict(q_len=-1), False, 2), (dict(scale=-1.0), False, 3),
    (dict(scale=float("inf")), False, 3), (dict(scale=float("nan")), False, 3), (dict(d_qk=96, d_v=96), False, 4),
    (dict(d_qk=128, d_v=64), False, 4), (dict(out_dtype=sdpa.F16), False, 4), (dict(descale=(1.0, -2.0, 1.0)), False, 3),
    (dict(q_len=2), True, 2), (dict(d_qk=96, d_v=96), True, 4), (dict(in_dtype=sdpa.FP8_E4M3), True, 4),
])
def test_validation_errors(over, decode, code):
    base = inputs.WORKLOADS["splitkv_decode_bf16" if decode else "gqa_causal_prefill_bf16"]
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.plan(_problem(base, **over), decode=decode)
    assert ei.value.status == code
    assert sdpa.load().sdpa_last_error() != b""


def test_null_and_workspace_errors_before_any_launch():
    """These return before touching the GPU, so they run on the CPU."""
    import ctypes

    lib = sdpa.load()
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    pr = _problem(w)
    null = ctypes.c_void_p(0)
    assert lib.sdpa_prefill_fwd(None, null, null, null, null, null, null, 0, null) == 1
    assert lib.sdpa_prefill_fwd(ctypes.byref(pr), null, null, null, null, null, null, 0, null) == 1
    mis = ctypes.c_void_p(0x1008)
    assert lib.sdpa_prefill_fwd(ctypes.byref(pr), mis, mis, mis, mis, null, null, 0, null) == 5
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    dp = _problem(dw)
    a = ctypes.c_void_p(0x1000)
    need = lib.sdpa_decode_workspace_bytes(ctypes.byref(dp), 0)
    assert need > 0
    assert lib.sdpa_decode_fwd(ctypes.byref(dp), a, a, a, a, null, 0, a, need - 16, null) == 6
    assert lib.sdpa_decode_fwd(ctypes.byref(dp), a, a, a, a, null, 0, null, need, null) in (5, 6)
    # empty problems are successful no-ops with no pointer checks
    empty = _problem(w, q_len=0)
    assert lib.sdpa_prefill_fwd(ctypes.byref(empty), null, null, null, null, null, null, 0, null) == 0


def test_paged_decode_argument_errors_before_any_launch():
    """sdpa_decode_paged_fwd checks the page geometry, alignment and workspace
    on the host and returns before enqueuing anything (so this runs on the CPU)."""
    import ctypes

    lib = sdpa.load()
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    dp = _problem(dw)
    null = ctypes.c_void_p(0)
    a = ctypes.c_void_p(0x1000)
    need = lib.sdpa_decode_workspace_bytes(ctypes.byref(dp), 0)
    pages = dw.kv_len // 64

    def call(problem=dp, table=a, lens=null, num_pages=dw.batch * pages, page_size=64, per_seq=pages,
             ws=a, ws_bytes=need):
        return lib.sdpa_decode_paged_fwd(None if problem is None else ctypes.byref(problem), a, a, a, lens, table,
                                         num_pages, page_size, per_seq, a, null, 0, ws, ws_bytes, null)

    assert call(problem=None) == 1
    assert call(page_size=48) == 2                      # not 8, 16 or a multiple of the 32-key block
    assert b"page_size" in lib.sdpa_last_error()
    assert call(page_size=0) == 2
    assert call(page_size=24) == 2
    assert call(page_size=4) == 2
    assert call(page_size=16, per_seq=dw.kv_len // 16, num_pages=dw.batch * dw.kv_len // 16, ws_bytes=need - 16) == 6
    assert call(per_seq=pages - 1) == 2                 # table row shorter than kv_len
    assert call(num_pages=0) == 2
    assert call(num_pages=2 ** 30) == 2                 # pool rows overflow int32
    assert call(table=ctypes.c_void_p(0x1002)) == 5     # table not 4-byte aligned
    assert call(lens=ctypes.c_void_p(0x1001)) == 5
    assert call(ws_bytes=need - 16) == 6
    # geometry is ignored without a table (dense variable-length form)
    assert call(table=null, page_size=48, ws_bytes=need - 16) == 6
    # an empty batch is a successful no-op
    assert call(problem=_problem(dw, batch=0), table=null, ws=null, ws_bytes=0) == 0


def test_paged_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    pool = torch.zeros(4, 64, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.decode_paged(q, pool, pool, page_table=torch.zeros(2, 2, dtype=torch.int32))  # host tensors
    with pytest.raises(ValueError):
        binding._check_caches(q, pool, pool[:3], dense=False)          # V pool smaller than K pool
    with pytest.raises(ValueError):
        binding._check_caches(q, pool, pool, dense=True)               # 4 dense rows for 2 sequences
    with pytest.raises(ValueError):
        binding._check_caches(q, pool[..., :64], pool, dense=False)    # head dim differs from q
    binding._check_caches(q, pool, pool, dense=False)


def test_cached_prefill_argument_errors_before_any_launch():
    import ctypes

    lib = sdpa.load()
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    null = ctypes.c_void_p(0)
    a = ctypes.c_void_p(0x1000)

    def call(problem, cache_len=1024, cap=1024, kc=a, k=a, q=a):
        return lib.sdpa_prefill_cached_fwd(None if problem is None else ctypes.byref(problem), q, kc, kc, cache_len,
                                           cap, k, k, a, null, null, 0, null)

    pr = _problem(w, q_len=512, kv_len=512)
    assert call(None) == 1
    assert call(pr, cache_len=-1) == 2
    assert call(pr, cache_len=100, cap=99) == 2
    assert call(_problem(w, q_len=600, kv_len=512)) == 2          # causal: more queries than new keys
    assert b"q_len" in lib.sdpa_last_error()
    assert call(pr, kc=null) == 1
    assert call(pr, kc=ctypes.c_void_p(0x1008)) == 5
    assert call(_problem(w, q_len=512, kv_len=512, in_dtype=sdpa.FP8_E4M3, d_qk=192)) == 4
    assert call(_problem(w, q_len=0, kv_len=512)) == 0              # no queries: a no-op
    # nothing cached: the plain prefill's checks (k_cache may be NULL)
    assert call(pr, cache_len=0, cap=0, kc=null, q=null) == 1



def test_split_prefill_workspace_errors_before_any_launch():
    """A split plan with a large enough workspace checks its alignment before
    any launch; the cached form likewise."""
    import ctypes

    lib = sdpa.load()
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    a, null = ctypes.c_void_p(0x1000), ctypes.c_void_p(0)
    pr = _problem(w, q_len=16, kv_len=8192)
    need = lib.sdpa_prefill_workspace_bytes(ctypes.byref(pr))
    assert need > 0
    odd = ctypes.c_void_p(0x1008)
    assert lib.sdpa_prefill_fwd(ctypes.byref(pr), a, a, a, a, null, odd, need, null) == 5
    assert b"workspace" in lib.sdpa_last_error()
    chunk = _problem(w, q_len=16, kv_len=16)
    cneed = lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(chunk), 8176)
    assert cneed == need
    assert lib.sdpa_prefill_cached_fwd(ctypes.byref(chunk), a, a, a, 8176, 8192, a, a, a, null, odd, cneed,
                                       null) == 5


def test_mask_convert_argument_errors_before_any_launch():
    import ctypes

    lib = sdpa.load()
    a, null = ctypes.c_void_p(0x1000), ctypes.c_void_p(0)
    assert lib.sdpa_mask_convert(a, a, -1, sdpa.BF16, null) == 2
    assert lib.sdpa_mask_convert(a, a, 16, sdpa.FP8_E4M3, null) == 4
    assert lib.sdpa_mask_convert(null, a, 16, sdpa.F16, null) == 1
    assert lib.sdpa_mask_convert(ctypes.c_void_p(0x1001), a, 16, sdpa.F16, null) == 5
    assert lib.sdpa_mask_convert(null, null, 0, sdpa.F16, null) == 0      # empty: a no-op


def test_hbm_read_probe_argument_errors_before_any_launch():
    import ctypes

    import torch

    lib = sdpa.load()
    a, null = ctypes.c_void_p(0x1000), ctypes.c_void_p(0)
    assert lib.sdpa_hbm_read_probe(a, -16, a, null) == 2
    assert lib.sdpa_hbm_read_probe(a, 24, a, null) == 2                 # not a multiple of 16
    assert lib.sdpa_hbm_read_probe(null, 16, a, null) == 1
    assert lib.sdpa_hbm_read_probe(a, 16, null, null) == 1
    assert lib.sdpa_hbm_read_probe(ctypes.c_void_p(0x1008), 16, a, null) == 5
    assert lib.sdpa_hbm_read_probe(a, 16, ctypes.c_void_p(0x1002), null) == 5
    assert lib.sdpa_hbm_read_probe(null, 0, null, null) == 0            # empty: a no-op
    with pytest.raises(ValueError):
        sdpa.hbm_read_probe(torch.zeros(16))                            # host tensor


def test_masked_prefill_argument_errors_before_any_launch():
    import ctypes

    lib = sdpa.load()
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    a, null = ctypes.c_void_p(0x1000), ctypes.c_void_p(0)
    pr = _problem(w, causal=False)

    def call(problem=pr, sb=0, sh=0, row=1024, mask=a):
        return lib.sdpa_prefill_masked_fwd(None if problem is None else ctypes.byref(problem), a, a, a, mask, sb, sh,
                                           row, a, null, null)

    assert call(None) == 1
    assert call(row=1000) == 2                       # row stride below kv_len
    assert call(row=1028) == 2                       # not a multiple of 8
    assert call(sb=-8) == 2
    assert call(sh=12) == 2
    assert call(mask=null) == 1
    assert call(mask=ctypes.c_void_p(0x1008)) == 5
    assert call(_problem(w, causal=False, out_dtype=sdpa.F16)) == 4     # output type differs from the input's
    assert call(_problem(w, causal=False, q_len=0)) == 0


def test_binding_rejects_mismatched_tensors():
    """The binding checks every tensor the kernels index before any launch:
    one dtype and device for q/k/v, consistent batch / head / dim, and the
    exact shape and dtype of a caller's out / lse.  The CPU tensors here fail
    the device check first, so a second set of checks runs through the
    shape/dtype validators directly."""
    import torch

    from attention_flash_sdpa_amd import binding as bd

    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        sdpa.prefill(q, k, v)
    with pytest.raises(ValueError, match="batch"):
        bd._check_prefill_shapes(q, torch.zeros(2, 16, 2, 64), torch.zeros(2, 16, 2, 64))
    with pytest.raises(ValueError, match="head dim"):
        bd._check_prefill_shapes(q, torch.zeros(1, 16, 2, 128), torch.zeros(1, 16, 2, 64))
    with pytest.raises(ValueError, match="does not match k"):
        bd._check_prefill_shapes(q, k, torch.zeros(1, 15, 2, 64))
    bd._check_prefill_shapes(q, k, v)
    with pytest.raises(ValueError, match="must be"):
        bd._check_output("out", torch.zeros(1, 8, 4, 32, dtype=torch.bfloat16), (1, 8, 4, 64), (torch.bfloat16,),
                         q.device)
    with pytest.raises(ValueError, match="dtype"):
        bd._check_output("lse", torch.zeros(1, 4, 8, dtype=torch.float16), (1, 4, 8), (torch.float32,), q.device)
    with pytest.raises(ValueError, match="contiguous"):
        bd._check_output("lse", torch.zeros(1, 8, 4).transpose(1, 2), (1, 4, 8), (torch.float32,), q.device)
    assert bd._out_dtypes(q) == (torch.bfloat16,)
    assert set(bd._out_dtypes(q.to(torch.float8_e4m3fn))) == {torch.bfloat16, torch.float16}
