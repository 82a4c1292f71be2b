"""The no-allocation decode entry point (sdpa_decode_fwd_noalloc) against the
workspace entry point (sdpa_decode_fwd) on the same inputs: two calls in a
row, the second with a smaller problem, each compared element by element
(the two paths run the same kernels with the same split count, so the outputs
are bit-identical) and against the fp64 oracle within the 2e-2 bar."""
import sys

import numpy as np
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


def _case(dev, oracle_mod, B, Hq, Hkv, Sk, D, dt, seed, num_splits=0):
    _say(f"no-alloc decode B={B} Hq={Hq} Hkv={Hkv} Sk={Sk} D={D} {dt} splits={num_splits or 'planner'}")
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    want = sdpa.decode(qd, kd, vd, num_splits=num_splits)
    want_lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sdpa.decode(qd, kd, vd, num_splits=num_splits, lse=want_lse)
    got = torch.full((B, Hq, D), float("nan"), dtype=dt, device=dev)
    got_lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.decode_noalloc(qd, kd, vd, num_splits=num_splits, out=got, lse=got_lse)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "outputs differ from sdpa_decode_fwd"
    assert torch.equal(got_lse, want_lse), "lse differs from sdpa_decode_fwd"
    ref = oracle_mod.sdpa(q.reshape(B, 1, Hq, D), k, v, scale=1 / D ** 0.5, causal=False)["out"][:, 0]
    err = float(np.abs(got.double().cpu().numpy() - ref).max())
    _say(f"  max_abs vs oracle {err:.3e}")
    assert err <= 2e-2


def test_noalloc_decode_two_calls_second_smaller(dev, oracle_mod):
    # the decode workload's head layout, then a smaller one: the second call
    # reuses the static scratch the first one left filled
    _case(dev, oracle_mod, 4, 32, 8, 2048, 128, torch.bfloat16, 11)
    _case(dev, oracle_mod, 2, 8, 2, 333, 64, torch.float16, 12)


def test_noalloc_decode_forced_splits_and_size_limit(dev, oracle_mod):
    _case(dev, oracle_mod, 3, 16, 4, 1000, 128, torch.bfloat16, 13, num_splits=40)
    _case(dev, oracle_mod, 1, 4, 1, 64, 64, torch.bfloat16, 14, num_splits=1)
    # partials beyond the 64 MiB scratch are refused before any launch
    B, Hq, Hkv, D = 64, 64, 8, 128
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, 64, Hkv, D, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sdpa.SdpaError, match="WORKSPACE"):
        sdpa.decode_noalloc(q, k, k, num_splits=2048)
