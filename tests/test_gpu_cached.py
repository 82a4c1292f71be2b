"""GPU parity of the cached-KV (chunked) prefill (``sdpa_prefill_cached_fwd``)
against the fp64 oracle ``oracle.cached.prefill_cached``, with and without
the keys split across workgroups.

Cache tensors carry slots past cache_len filled with NaN, so a read of a slot
that holds no key shows in the output.  Bar as for the plain prefill: no NaN,
max |gpu - oracle| <= 2e-2 on O, the lse bound of the plain tests.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_flash_sdpa_amd as sdpa

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


def _draw(B, Sq, Sc, cap, Sk, Hq, Hkv, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Sq, Hq, D, generator=g).to(dt)
    kc = torch.randn(B, cap, Hkv, D, generator=g).to(dt)
    vc = torch.randn(B, cap, Hkv, D, generator=g).to(dt)
    kc[:, Sc:] = float("nan")
    vc[:, Sc:] = float("nan")
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    return q, kc, vc, k, v


def _case(dev, q, kc, vc, k, v, *, cache_len, causal, scale):
    from oracle import cached as oc

    B, Sq, Hq, _ = q.shape
    out = torch.full((B, Sq, Hq, v.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    # a key range split across workgroups keeps partials in the workspace:
    # NaN bytes first, so a partial row left unwritten shows in the output
    n = sdpa.prefill_cached_workspace_bytes(q, k, v, cache_len=cache_len, causal=causal)
    ws = torch.full((max(n, 16),), 255, dtype=torch.uint8, device=dev)
    sdpa.prefill_cached(*(t.to(dev) for t in (q, kc, vc, k, v)), cache_len=cache_len, causal=causal, scale=scale,
                        out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ref = oc.prefill_cached(q, kc, vc, k, v, cache_len=cache_len, scale=scale, causal=causal)
    got = out.double().cpu().numpy()
    nan = int(np.isnan(got).sum())
    err = float(np.abs(got - ref["out"]).max())
    _say(f"  out: nan={nan} max_abs={err:.3e}")
    assert nan == 0 and err <= TOL16, (nan, err)
    gl = lse.double().cpu().numpy()
    want = ref["lse"]
    assert np.array_equal(np.isneginf(gl), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.abs(gl[fin] - want[fin]).max(initial=0) <= _lse_tol(q.dtype)
    return out


CASES = [
    # B, Sq, cache_len, cache_cap, new keys, Hq, Hkv, D, dtype, causal
    (1, 128, 192, 256, 128, 8, 2, 128, torch.bfloat16, True),    # cache a whole number of blocks
    (2, 100, 150, 160, 100, 8, 2, 128, torch.bfloat16, True),    # a block straddles cache and new keys
    (1, 64, 30, 30, 80, 4, 4, 64, torch.float16, True),          # cache shorter than a block, Sq < new keys
    (2, 77, 300, 300, 77, 28, 4, 128, torch.bfloat16, False),    # full attention over cache + chunk
    (1, 17, 1000, 1024, 17, 32, 8, 128, torch.bfloat16, True),   # short chunk, long cache
    (1, 1, 500, 512, 1, 8, 1, 64, torch.bfloat16, True),         # one new token
    (1, 200, 5, 5, 200, 4, 2, 64, torch.float16, True),          # a few cached keys
    (1, 40, 700, 700, 0, 8, 2, 128, torch.bfloat16, False),      # no new keys: the cache only
    (2, 96, 64, 64, 40, 8, 4, 64, torch.float16, False),         # full attention, more queries than new keys
    (1, 300, 4000, 4096, 300, 16, 2, 128, torch.float16, True),  # fp16, d 128, long cache, 8 query heads per KV head
    # cache and key counts multiples of the rows one 1 KiB fill covers (4 at
    # d 128, 8 at d 64), with a block straddling the two: the scalar-base form
    (1, 60, 100, 128, 60, 8, 2, 128, torch.bfloat16, True),
    (1, 72, 200, 256, 72, 8, 2, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("variant", ["", "narrow1", "narrow2", "occ2", "split4", "kvsplit", "kvsplit1"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_q{c[1]}_c{c[2]}of{c[3]}_k{c[4]}_h{c[5]}x{c[6]}_d{c[7]}_"
                                             f"{'causal' if c[9] else 'full'}" for c in CASES])
def test_cached_prefill(dev, case, variant, prefill_variant):
    B, Sq, Sc, cap, Sk, Hq, Hkv, D, dt, causal = case
    if variant:
        prefill_variant(variant)
    _say(f"cached prefill B={B} q={Sq} cache={Sc}/{cap} new={Sk} Hq={Hq} Hkv={Hkv} D={D} {dt} causal={causal} "
         f"variant={variant or 'default'}")
    q, kc, vc, k, v = _draw(B, Sq, Sc, cap, Sk, Hq, Hkv, D, dt, Sq + 7 * Sc + Sk)
    _case(dev, q, kc, vc, k, v, cache_len=Sc, causal=causal, scale=1 / math.sqrt(D))


def test_chunked_prefill_of_a_sequence(dev):
    """A 1000-token sequence in chunks of 256, 256, 300 and 188 tokens, each
    over the earlier tokens as its cache (the sequence's own K/V buffer),
    against the oracle, and against the one-shot causal prefill."""
    from oracle import cached as oc

    B, S, Hq, Hkv, D = 1, 1000, 16, 4, 128
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, S, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, S, Hkv, D, generator=g).to(torch.bfloat16)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    whole = sdpa.prefill(qd, kd, vd, causal=True)
    lo = 0
    for n in (256, 256, 300, 188):
        hi = lo + n
        _say(f"chunk [{lo}, {hi})")
        o = sdpa.prefill_cached(qd[:, lo:hi].contiguous(), kd, vd, kd[:, lo:hi].contiguous(),
                                vd[:, lo:hi].contiguous(), cache_len=lo, causal=True)
        torch.cuda.synchronize()
        ref = oc.prefill_cached(q[:, lo:hi], k, v, k[:, lo:hi], v[:, lo:hi], cache_len=lo, scale=1 / math.sqrt(D),
                                causal=True)
        assert np.abs(o.double().cpu().numpy() - ref["out"]).max() <= TOL16
        assert (o.float() - whole[:, lo:hi].float()).abs().max().item() <= TOL16
        lo = hi


def test_cached_prefill_chunk_workload_full_size(dev):
    """A 512-token chunk over a 3584-token cache (4096 keys in all), 32 query /
    8 KV heads, head dim 128, bf16, causal: every row against the oracle."""
    B, Sq, Sc, Hq, Hkv, D = 1, 512, 3584, 32, 8, 128
    _say("cached prefill chunk workload 512 over 3584")
    q, kc, vc, k, v = _draw(B, Sq, Sc, Sc, Sq, Hq, Hkv, D, torch.bfloat16, 1006)
    _case(dev, q, kc, vc, k, v, cache_len=Sc, causal=True, scale=1 / math.sqrt(D))


@pytest.mark.parametrize("cache_len,new", [(8176, 16), (8000, 64), (5000, 3)])
def test_short_chunk_over_long_cache_splits(dev, cache_len, new):
    """A short chunk over a long cache: the planner spreads each tile's keys
    over several workgroups (the partials merged by the combine kernel)."""
    B, Sq, Hq, Hkv, D = 1, min(new, 16), 32, 8, 128
    _say(f"split cached prefill: {Sq} queries, {new} new keys over {cache_len} cached")
    q, kc, vc, k, v = _draw(B, Sq, cache_len, cache_len + 7, new, Hq, Hkv, D, torch.bfloat16, cache_len + new)
    assert sdpa.prefill_cached_workspace_bytes(q, k, v, cache_len=cache_len, causal=True) > 0
    _case(dev, q, kc, vc, k, v, cache_len=cache_len, causal=True, scale=1 / math.sqrt(D))


def test_cached_prefill_rejects_more_queries_than_new_keys(dev):
    q = torch.zeros(1, 10, 4, 64, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(1, 32, 2, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.prefill_cached(q, kc, kc, k, k, cache_len=32, causal=True)
    assert ei.value.status == 2
