"""HIP-graph capture of the C-ABI calls (the way bench.py times them).

The library allocates, frees and synchronizes nothing, so a caller may capture
its launches into a graph.  Each replay here is checked bit for bit against
the eager call on the same inputs, with eager work and synchronizations
between the replays, and the graph's output buffer cleared before each replay
so that a replay which did nothing cannot pass.
"""
import sys

import pytest
import torch

import attention_flash_sdpa_amd as sdpa
from attention_flash_sdpa_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sdpa.load()
    return torch.device("cuda:0")


def _replays_match(dev, call, out, n_calls, replays=3):
    torch.cuda.synchronize()
    call(0)
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            call(i)
    for r in range(replays):
        out.zero_()
        scratch = torch.randn(1 << 20, device=dev)        # eager work between replays
        scratch.mul_(2.0).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, want)
        diff = (out.float() - want.float()).abs()
        _say(f"  replay {r}: bit-identical={same} differing={int((diff > 0).sum())} max_abs_diff={float(diff.max()):.3e}")
        assert same, f"replay {r} differs from the eager call"


def test_prefill_graph_replay(dev):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=200, kv_len=333)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty(w.batch, 200, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.batch, w.head_q, 200, dtype=torch.float32, device=dev)
    _say("prefill graph: causal GQA bf16 q 200 kv 333")
    _replays_match(dev, lambda i: sdpa.prefill(qd, kd, vd, scale=w.scale, causal=True, out=out, lse=lse), out, 2)


def test_split_prefill_graph_replay(dev):
    """A 16-token chunk over 8,192 keys: the split kernel and the combine
    through one workspace, captured and replayed; lse checked too."""
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=16, kv_len=8192)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    n = sdpa.prefill_workspace_bytes(qd, kd, vd, causal=True)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    out = torch.empty(w.batch, 16, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.batch, w.head_q, 16, dtype=torch.float32, device=dev)
    _say("split prefill graph: causal GQA bf16 q 16 kv 8192")

    def call(i):
        sdpa.prefill(qd, kd, vd, scale=w.scale, causal=True, out=out, lse=lse, workspace=ws)

    _replays_match(dev, call, out, 2)
    lse_want = lse.clone()
    lse.zero_()
    call(0)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse_want)


def test_decode_graph_replay(dev):
    w = inputs.WORKLOADS["splitkv_decode_bf16"]
    q, k, v, _ = inputs.make_qkv(w, kv_len=1500)
    qd = q.reshape(w.batch, w.head_q, w.d_qk).to(dev)
    kd, vd = k.to(dev), v.to(dev)
    out = torch.empty(w.batch, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    ws = sdpa.decode_workspace(qd, kd, vd)
    _say("decode graph: B16 32/8 heads kv 1500")
    _replays_match(dev, lambda i: sdpa.decode(qd, kd, vd, scale=w.scale, out=out, workspace=ws), out, 2)


def test_paged_decode_graph_replay(dev):
    d = inputs.WORKLOADS["splitkv_decode_bf16"]
    q, k, v, _ = inputs.make_qkv(d, kv_len=900)
    qd = q.reshape(d.batch, d.head_q, d.d_qk).to(dev)
    kp, vp, table = inputs.paginate(k, v, 16, seed=3, spare_pages=4)
    lens = inputs.length_mix(d.batch, 900, seed=4).to(dev)
    kpd, vpd, td = kp.to(dev), vp.to(dev), table.to(dev)
    out = torch.empty(d.batch, d.head_q, d.d_v, dtype=torch.bfloat16, device=dev)
    ws = sdpa.decode_workspace(qd, kpd, vpd, kv_len=900)
    _say("paged decode graph: 16-key pages, mixed lengths")
    _replays_match(dev, lambda i: sdpa.decode_paged(qd, kpd, vpd, page_table=td, seq_lens=lens, kv_len=900,
                                                    out=out, workspace=ws), out, 2)


def test_cached_prefill_graph_replay(dev):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=128, kv_len=400)
    qd = q.to(dev)
    kc, vc = k[:, :272].contiguous().to(dev), v[:, :272].contiguous().to(dev)
    kn, vn = k[:, 272:].contiguous().to(dev), v[:, 272:].contiguous().to(dev)
    out = torch.empty(w.batch, 128, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    _say("cached prefill graph: 128 queries over 272 cached keys")
    _replays_match(dev, lambda i: sdpa.prefill_cached(qd, kc, vc, kn, vn, cache_len=272, causal=True, out=out),
                   out, 2)


def test_mask_convert_and_masked_prefill_graph_replay(dev):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=96, kv_len=160)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    keep = (torch.rand(1, 1, 96, 160, generator=torch.Generator().manual_seed(5)) < 0.7).to(dev)
    add = torch.empty(1, 1, 96, 160, dtype=torch.bfloat16, device=dev)
    out = torch.empty(w.batch, 96, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)

    def call(i):
        sdpa.mask_convert(keep, out=add)
        sdpa.prefill_masked(qd, kd, vd, add, out=out)

    _say("mask conversion + masked prefill graph")
    _replays_match(dev, call, out, 2)
