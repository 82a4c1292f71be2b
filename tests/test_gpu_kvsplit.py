"""GPU parity of the prefill split across workgroups (plan.kv_splits > 1:
fp32 partials per key range in the caller's workspace, merged by the combine
kernel) against the fp64 oracle, through ``sdpa_prefill_fwd``.

The shapes are the ones the planner splits on its own (short query chunks over
long key sequences, too few query tiles to fill the GPU) plus forced splits
("kvsplit") where some workgroups' key ranges hold no key.  The workspace is
filled with NaN bytes first, so a partial row the kernel fails to write shows
in the output.  Bar as for the plain prefill: no NaN, max |gpu - oracle| <=
2e-2 on O, 1e-3 on lse."""
import math
import sys

import numpy as np
import pytest
import torch

import attention_flash_sdpa_amd as sdpa

pytestmark = pytest.mark.gpu

TOL16 = 2e-2
LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sdpa.load()
    return torch.device("cuda:0")


def _draw(B, Sq, Sk, Hq, Hkv, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Sq, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    return q, k, v


def _plan(q, k, causal):
    B, Sq, Hq, D = q.shape
    pr = sdpa.make_problem(batch=B, q_len=Sq, kv_len=k.shape[1], head_q=Hq, head_kv=k.shape[2], d_qk=D, d_v=D,
                           in_dtype=sdpa.BF16 if q.dtype == torch.bfloat16 else sdpa.F16,
                           out_dtype=sdpa.BF16 if q.dtype == torch.bfloat16 else sdpa.F16, causal=causal,
                           scale=1.0)
    return sdpa.plan(pr)


def _run(dev, q, k, v, *, causal, scale, workspace=None):
    B, Sq, Hq, _ = q.shape
    out = torch.full((B, Sq, Hq, v.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.prefill(*(t.to(dev) for t in (q, k, v)), scale=scale, causal=causal, out=out, lse=lse,
                 workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def _check(oracle_mod, q, k, v, out, lse, *, causal, scale):
    ref = oracle_mod.sdpa(q, k, v, scale=scale, causal=causal)
    got = out.double().cpu().numpy()
    nan = int(np.isnan(got).sum())
    err = float(np.abs(got - ref["out"]).max()) if got.size else 0.0
    _say(f"  out: nan={nan} max_abs={err:.3e}")
    assert nan == 0 and err <= TOL16, (nan, err)
    gl = lse.double().cpu().numpy()
    want = ref["lse"]
    assert np.array_equal(np.isneginf(gl), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.abs(gl[fin] - want[fin]).max(initial=0) <= LSE_TOL


def _poisoned_workspace(dev, q, k, v, causal):
    n = sdpa.prefill_workspace_bytes(q, k, v, causal=causal)
    return torch.full((max(n, 16),), 255, dtype=torch.uint8, device=dev), n  # 0xffffffff is a NaN


AUTO = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal
    (1, 16, 8192, 32, 8, 128, torch.bfloat16, True),   # a 16-token chunk over 8K keys: 16 splits
    (1, 16, 8192, 32, 8, 128, torch.bfloat16, False),
    (2, 5, 3000, 8, 2, 64, torch.float16, True),
    (1, 64, 4096, 8, 8, 128, torch.bfloat16, True),     # two 32-row tiles of one head per workgroup
    (1, 1, 2048, 4, 1, 128, torch.bfloat16, False),     # one query row
    (3, 40, 1999, 6, 3, 64, torch.bfloat16, True),      # ragged key count, odd group
    (1, 33, 4000, 2, 1, 128, torch.float16, False),     # a ragged second query tile
    (1, 8, 16384, 16, 4, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", AUTO, ids=[f"B{c[0]}_q{c[1]}_k{c[2]}_h{c[3]}x{c[4]}_d{c[5]}_{str(c[6])[6:]}_"
                                           f"{'c' if c[7] else 'f'}" for c in AUTO])
def test_planner_split_prefill(dev, oracle_mod, case):
    B, Sq, Sk, Hq, Hkv, D, dt, causal = case
    q, k, v = _draw(B, Sq, Sk, Hq, Hkv, D, dt, Sq * 7919 + Sk)
    p = _plan(q, k, causal)
    _say(f"split prefill {case}: kv_splits={p.kv_splits} ranges={p.num_splits} groups={p.num_groups}")
    assert p.kv_splits > 1  # the planner splits these shapes
    ws, n = _poisoned_workspace(dev, q, k, v, causal)
    assert n == p.workspace_bytes
    out, lse = _run(dev, q, k, v, causal=causal, scale=1 / math.sqrt(D), workspace=ws)
    _check(oracle_mod, q, k, v, out, lse, causal=causal, scale=1 / math.sqrt(D))


FORCED = [
    (1, 7, 5, 28, 4, 128, torch.bfloat16, True),      # one key block, empty rows, empty splits
    (2, 65, 33, 3, 1, 128, torch.float16, True),      # q_len > kv_len
    (1, 100, 300, 4, 2, 64, torch.bfloat16, True),
    (2, 3, 130, 16, 2, 128, torch.bfloat16, False),
]


@pytest.mark.parametrize("variant", ["kvsplit", "kvsplit1"])
@pytest.mark.parametrize("case", FORCED, ids=[f"B{c[0]}_q{c[1]}_k{c[2]}_h{c[3]}x{c[4]}_d{c[5]}_"
                                             f"{'c' if c[7] else 'f'}" for c in FORCED])
def test_forced_split_with_empty_ranges(dev, oracle_mod, case, variant, prefill_variant):
    prefill_variant(variant)
    B, Sq, Sk, Hq, Hkv, D, dt, causal = case
    q, k, v = _draw(B, Sq, Sk, Hq, Hkv, D, dt, Sq * 31 + Sk)
    p = _plan(q, k, causal)
    _say(f"forced split {case}: kv_splits={p.kv_splits} groups={p.num_groups}")
    assert p.kv_splits >= 2
    ws, _ = _poisoned_workspace(dev, q, k, v, causal)
    out, lse = _run(dev, q, k, v, causal=causal, scale=1 / math.sqrt(D), workspace=ws)
    _check(oracle_mod, q, k, v, out, lse, causal=causal, scale=1 / math.sqrt(D))


@pytest.mark.parametrize("variant", ["kvsplit", "kvsplit1"])
def test_forced_split_with_no_keys(dev, variant, prefill_variant):
    prefill_variant(variant)
    q = torch.randn(2, 5, 4, 128).to(torch.bfloat16)
    k = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16)
    ws, n = _poisoned_workspace(dev, q, k, k, False)
    assert n > 0
    out, lse = _run(dev, q, k, k, causal=False, scale=0.1, workspace=ws)
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_without_workspace_the_same_problem_runs_unsplit(dev, oracle_mod):
    """An empty workspace: the call plans without the split and still
    succeeds, within the same bar."""
    B, Sq, Sk, Hq, Hkv, D = 1, 16, 8192, 32, 8, 128
    q, k, v = _draw(B, Sq, Sk, Hq, Hkv, D, torch.bfloat16, 77)
    assert _plan(q, k, True).kv_splits > 1
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    out0, lse0 = _run(dev, q, k, v, causal=True, scale=1 / math.sqrt(D), workspace=empty)
    _check(oracle_mod, q, k, v, out0, lse0, causal=True, scale=1 / math.sqrt(D))
    out1, lse1 = _run(dev, q, k, v, causal=True, scale=1 / math.sqrt(D))
    assert (out0.float() - out1.float()).abs().max().item() <= TOL16
    assert (lse0 - lse1).abs().max().item() <= LSE_TOL


def test_split_constant_values_and_repeat(dev, oracle_mod):
    """Constant V gives that constant exactly through the combine as well, and
    two calls on a reused workspace give identical bits."""
    B, Sq, Sk, Hq, Hkv, D = 1, 16, 8192, 32, 8, 128
    q, k, v = _draw(B, Sq, Sk, Hq, Hkv, D, torch.bfloat16, 78)
    vc = torch.full_like(v, 0.75)
    ws, _ = _poisoned_workspace(dev, q, k, vc, True)
    out, _ = _run(dev, q, k, vc, causal=True, scale=0.1, workspace=ws)
    assert torch.equal(out.float().cpu(), torch.full((B, Sq, Hq, D), 0.75))
    a, la = _run(dev, q, k, v, causal=True, scale=1 / math.sqrt(D), workspace=ws)
    b, lb = _run(dev, q, k, v, causal=True, scale=1 / math.sqrt(D), workspace=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
