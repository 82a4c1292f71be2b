"""GPU parity of the prefill with a full additive mask
(``sdpa_prefill_masked_fwd``) against the fp64 oracle
``oracle.mask.prefill_masked``.  Bar as for the plain prefill: no NaN where
the oracle has none, max |gpu - oracle| <= 2e-2 on O, the lse bound of the
plain tests, and O = 0 / lse = -inf exactly for fully masked rows."""
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


def _padded(m, dev):
    """Device copy of mask m [Bm, Hm, Sq, Sk] in rows padded to a multiple of
    8 elements (padding = NaN, which the kernel must never use), sliced back
    to Sk."""
    Sk = m.shape[-1]
    W = max(8, -(-Sk // 8) * 8)
    buf = torch.full((*m.shape[:3], W), float("nan"), dtype=m.dtype)
    buf[..., :Sk] = m
    return buf.to(dev)[..., :Sk]


def _case(dev, q, k, v, mask, *, causal, scale, rows=None):
    from oracle import mask as om

    B, Sq, Hq, _ = q.shape
    out = torch.full((B, Sq, Hq, v.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.prefill_masked(q.to(dev), k.to(dev), v.to(dev), _padded(mask, dev), scale=scale, causal=causal, out=out,
                        lse=lse)
    torch.cuda.synchronize()
    ref = om.prefill_masked(q, k, v, mask, scale=scale, causal=causal)
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
    return out, ref


def _draw(B, Sq, Sk, Hq, Hkv, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Sq, Hq, D, generator=g).to(dt), torch.randn(B, Sk, Hkv, D, generator=g).to(dt),
            torch.randn(B, Sk, Hkv, D, generator=g).to(dt), g)


CASES = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal, mask batch dim, mask head dim, kind
    (1, 64, 128, 4, 2, 128, torch.bfloat16, False, 1, 4, "bias"),
    (2, 100, 77, 8, 2, 64, torch.float16, True, 1, 8, "keep"),
    (1, 333, 1000, 4, 4, 128, torch.bfloat16, True, 1, 1, "bias"),
    (2, 17, 5, 2, 1, 64, torch.bfloat16, False, 2, 1, "keep"),
    (3, 50, 300, 6, 3, 128, torch.float16, False, 3, 6, "bias+keep"),
    (1, 200, 150, 4, 1, 64, torch.bfloat16, True, 1, 1, "bias"),      # causal, more queries than keys: empty rows
    (2, 257, 513, 8, 8, 128, torch.bfloat16, False, 2, 8, "keep"),    # ragged rows and keys, per-(batch, head) mask
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_q{c[1]}_k{c[2]}_h{c[3]}x{c[4]}_d{c[5]}_"
                                             f"{'causal' if c[7] else 'full'}_m{c[8]}x{c[9]}_{c[10]}" for c in CASES])
def test_masked_prefill(dev, case):
    from oracle import mask as om

    B, Sq, Sk, Hq, Hkv, D, dt, causal, mb, mh, kind = case
    _say(f"masked prefill B={B} q={Sq} k={Sk} Hq={Hq} Hkv={Hkv} D={D} {dt} causal={causal} mask {mb}x{mh} {kind}")
    q, k, v, g = _draw(B, Sq, Sk, Hq, Hkv, D, dt, Sq + Sk)
    m = torch.zeros(mb, mh, Sq, Sk)
    if "bias" in kind:
        m += torch.randn(mb, mh, Sq, Sk, generator=g) * 2
    if "keep" in kind:
        keep = torch.rand(mb, mh, Sq, Sk, generator=g) < 0.7
        keep[..., 0] = True
        add = om.mask_convert(keep.numpy().astype(np.uint8), "f16").astype(np.float32)
        m += torch.from_numpy(add)
    _case(dev, q, k, v, m.to(dt), causal=causal, scale=1 / math.sqrt(D))


def test_fully_masked_rows_and_zero_mask(dev):
    """Rows whose mask is -inf everywhere give O = 0, lse = -inf; a zero mask
    gives the plain prefill's result."""
    q, k, v, g = _draw(1, 40, 90, 4, 2, 128, torch.bfloat16, 3)
    m = torch.zeros(1, 1, 40, 90)
    m[:, :, 5] = float("-inf")
    m[:, :, 31] = float("-inf")
    out, _ = _case(dev, q, k, v, m.to(torch.bfloat16), causal=False, scale=0.1)
    assert (out[0, 5].float() == 0).all() and (out[0, 31].float() == 0).all()
    plain = sdpa.prefill(q.to(dev), k.to(dev), v.to(dev), scale=0.1)
    zero = sdpa.prefill_masked(q.to(dev), k.to(dev), v.to(dev), _padded(torch.zeros(1, 1, 40, 90).bfloat16(), dev),
                               scale=0.1)
    torch.cuda.synchronize()
    assert (plain.float() - zero.float()).abs().max().item() <= TOL16


def test_masked_prefill_workload_full_size(dev):
    """32 query / 8 KV heads, 1024 x 1024, head dim 128, bf16, a per-head
    additive bias (a linear distance penalty with a per-head slope plus
    noise), every row against the oracle."""
    B, S, Hq, Hkv, D = 1, 1024, 32, 8, 128
    q, k, v, g = _draw(B, S, S, Hq, Hkv, D, torch.bfloat16, 1008)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    slope = 2.0 ** (-torch.arange(1, Hq + 1) / 4.0)
    m = -(slope[:, None, None] * (i - j).abs()[None]) + 0.1 * torch.randn(Hq, S, S, generator=g)
    _say("masked prefill workload 1024 x 1024, per-head bias")
    _case(dev, q, k, v, m[None].to(torch.bfloat16), causal=False, scale=1 / math.sqrt(D))


def test_masked_prefill_rejects_bad_strides(dev):
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 12, 2, 64, dtype=torch.bfloat16, device=dev)
    m = torch.zeros(1, 1, 8, 12, dtype=torch.bfloat16, device=dev)     # row stride 12: not a multiple of 8
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.prefill_masked(q, k, k, m)
    assert ei.value.status == 2


def test_masked_prefill_without_keys(dev):
    q = torch.randn(1, 20, 4, 64).to(torch.bfloat16).to(dev)
    k = torch.empty(1, 0, 2, 64, dtype=torch.bfloat16, device=dev)
    m = torch.empty(1, 1, 20, 0, dtype=torch.bfloat16, device=dev)
    out = torch.full((1, 20, 4, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(1, 4, 20, device=dev)
    sdpa.prefill_masked(q, k, k, m, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
