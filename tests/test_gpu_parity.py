"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar (per output element, after counting NaNs first, as "xe2-sdp-kernels",
section "Correctness testing", advises): zero NaNs and max |gpu - oracle| <=
2e-2 for fp16/bf16 inputs.  Every input comes from the seeded generator in
attention_flash_sdpa_amd.inputs.
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
TOL8 = 6e-2


def _lse_tol(dtype):
    """The row sum l is taken over the fp32 probabilities (before their rounding
    to the MFMA operand type), so lse carries fp32 rounding only: the
    sequential sum of n terms is within n * 2^-24 relative, and 1e-3 covers
    rows of 16K keys."""
    return 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sdpa.load()
    return torch.device("cuda:0")


def _compare(got, want, tol, what):
    got = got.detach().double().cpu().numpy()
    nan = int(np.isnan(got).sum())
    err = np.abs(got - want)
    worst = float(err.max()) if err.size else 0.0
    _say(f"  {what}: nan={nan} max_abs={worst:.3e} mean_abs={float(err.mean()) if err.size else 0:.3e}")
    assert nan == 0, f"{what}: {nan} NaNs"
    assert worst <= tol, f"{what}: max abs err {worst} > {tol} at {np.unravel_index(err.argmax(), err.shape)}"
    return worst


def _prefill_case(dev, oracle_mod, q, k, v, *, causal, scale, tol=TOL16, rows=None, check_lse=True, what="",
                  descale=(1.0, 1.0, 1.0)):
    B, Sq, Hq, _ = q.shape
    _say(f"prefill {what} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} scale={scale:.4g}")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    odt = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    out = torch.full((B, Sq, Hq, v.shape[-1]), float("nan"), dtype=odt, device=dev)
    sdpa.prefill(qd, kd, vd, scale=scale, causal=causal, out=out, lse=lse, descale=descale)
    torch.cuda.synchronize()
    ref = oracle_mod.sdpa(q, k, v, scale=scale, causal=causal, rows=rows, descale=descale)
    if rows is None:
        _compare(out, ref["out"], tol, "out")
        if check_lse:
            got = lse.double().cpu().numpy()
            want = ref["lse"]
            assert np.array_equal(np.isneginf(got), np.isneginf(want))
            fin = np.isfinite(want)
            assert np.abs(got[fin] - want[fin]).max(initial=0) <= _lse_tol(q.dtype)
    else:
        r = torch.as_tensor(rows)
        sel = out.cpu()[r[:, 0], r[:, 1], r[:, 2]]
        _compare(sel, ref["out"], tol, f"out[{len(rows)} sampled rows]")
        if check_lse:
            got = lse.cpu()[r[:, 0], r[:, 2], r[:, 1]].double().numpy()
            fin = np.isfinite(ref["lse"])
            assert np.array_equal(np.isneginf(got), np.isneginf(ref["lse"]))
            assert np.abs(got[fin] - ref["lse"][fin]).max(initial=0) <= _lse_tol(q.dtype)
    return out


def _sample_rows(B, Sq, Hq, n, seed):
    g = np.random.default_rng(seed)
    rows = [(b, i, h) for b in (0, B - 1) for i in (0, Sq - 1) for h in (0, Hq - 1)]
    rows += [(int(g.integers(B)), int(g.integers(Sq)), int(g.integers(Hq))) for _ in range(n)]
    return np.array(rows, dtype=np.int64)


# ------------------------------------------------------------------ workloads
def test_single_head_f16_128(dev, oracle_mod):
    w = inputs.WORKLOADS["single_head_f16_128"]
    q, k, v, _ = inputs.make_qkv(w)
    _prefill_case(dev, oracle_mod, q, k, v, causal=w.causal, scale=w.scale, what=w.name)


def test_gqa_causal_prefill_bf16(dev, oracle_mod):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    _prefill_case(dev, oracle_mod, q, k, v, causal=w.causal, scale=w.scale, what=w.name)


@pytest.mark.parametrize("variant", ["narrow1", "occ2", "split4"])
def test_gqa_causal_prefill_bf16_forms(dev, oracle_mod, variant, prefill_variant):
    """The full-size causal GQA workload through the other 32-row forms."""
    prefill_variant(variant)
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    _prefill_case(dev, oracle_mod, q, k, v, causal=w.causal, scale=w.scale, what=f"{w.name} {variant}")


def test_unaligned_full_bf16_reduced(dev, oracle_mod):
    """Same head layout and dtypes, lengths cut to 301 x 323 (several tiles and
    ragged tails in both dimensions) so every row is checked."""
    w = inputs.WORKLOADS["unaligned_full_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=301, kv_len=323)
    _prefill_case(dev, oracle_mod, q, k, v, causal=w.causal, scale=w.scale, what=w.name + " reduced")


def test_unaligned_full_bf16_full_size(dev, oracle_mod):
    """The full C3a workload, every one of its 56,056 rows against the oracle."""
    w = inputs.WORKLOADS["unaligned_full_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    _prefill_case(dev, oracle_mod, q, k, v, causal=w.causal, scale=w.scale, what=w.name)


def test_tiny_causal_bf16(dev, oracle_mod):
    w = inputs.WORKLOADS["tiny_causal_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    out = _prefill_case(dev, oracle_mod, q, k, v, causal=True, scale=w.scale, what=w.name)
    assert (out[:, :2].float().cpu() == 0).all()   # rows with no visible key


def test_mla_fp8_prefill_reduced(dev, oracle_mod):
    """fp8 e4m3 Q/K/V (per-tensor scales), d_qk 192 / d_v 128, bf16 output:
    8 heads with ragged lengths, causal and full, every row checked."""
    import dataclasses

    w = inputs.WORKLOADS["mla_fp8_causal_prefill"]
    for sq, sk, causal in ((333, 333, True), (200, 450, True), (130, 77, False), (77, 130, True)):
        small = dataclasses.replace(w, head_q=8, head_kv=8, q_len=sq, kv_len=sk)
        q, k, v, ds = inputs.make_qkv(small)
        _prefill_case(dev, oracle_mod, q, k, v, causal=causal, scale=w.scale, tol=TOL8, descale=ds,
                      what=f"fp8 {sq}x{sk}")


def test_mla_fp8_causal_prefill_full_size_sampled(dev, oracle_mod):
    w = inputs.WORKLOADS["mla_fp8_causal_prefill"]
    q, k, v, ds = inputs.make_qkv(w)
    rows = _sample_rows(w.batch, w.q_len, w.head_q, 4000, 11)
    extra = np.array([(0, i, h) for i in range(0, 9) for h in (0, 77)], dtype=np.int64)   # rows with few keys
    rows = np.concatenate([rows, extra])
    _prefill_case(dev, oracle_mod, q, k, v, causal=True, scale=w.scale, tol=TOL8, rows=rows, descale=ds,
                  what=w.name)


# ------------------------------------------------------------------ edge cases
EDGE = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal
    (1, 1, 1, 1, 1, 128, torch.bfloat16, False),
    (1, 1, 300, 4, 1, 128, torch.bfloat16, True),
    (2, 33, 65, 6, 2, 128, torch.bfloat16, True),
    (1, 65, 33, 3, 1, 128, torch.float16, True),      # q_len > kv_len: empty leading rows
    (1, 200, 200, 8, 8, 64, torch.bfloat16, True),
    (1, 97, 130, 2, 2, 64, torch.float16, False),
    (3, 64, 64, 16, 2, 128, torch.float16, True),
    (1, 129, 1, 7, 7, 128, torch.bfloat16, False),
    (1, 40, 520, 12, 4, 128, torch.bfloat16, True),
    (1, 256, 777, 5, 5, 64, torch.bfloat16, True),
    (1, 300, 130, 4, 2, 128, torch.bfloat16, True),   # 3 key blocks, many empty rows
    (1, 64, 192, 2, 1, 64, torch.float16, False),     # 3 whole key blocks
    (2, 96, 64, 2, 2, 128, torch.float16, True),      # one key block
    (1, 20, 150, 4, 2, 128, torch.bfloat16, True),    # key ranges past the last key
]


@pytest.mark.parametrize("variant", ["narrow1", "narrow2", "occ2", "split4", "kvsplit", "kvsplit1"])
@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}_q{c[1]}_k{c[2]}_h{c[3]}x{c[4]}_d{c[5]}_{str(c[6])[6:]}_{'c' if c[7] else 'f'}" for c in EDGE])
def test_prefill_edge_shapes(dev, oracle_mod, case, variant, prefill_variant):
    """Every edge shape through every 16-bit prefill kernel form: one wave per
    SIMD with one or two key ranges per workgroup (and both split across
    workgroups, with a combine), two waves per SIMD with one or four key
    ranges."""
    prefill_variant(variant)
    B, Sq, Sk, Hq, Hkv, D, dt, causal = case
    g = torch.Generator().manual_seed(Sq * 1000 + Sk)
    q = torch.randn(B, Sq, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    _prefill_case(dev, oracle_mod, q, k, v, causal=causal, scale=1 / math.sqrt(D))


def test_prefill_kv_len_zero(dev):
    q = torch.randn(2, 5, 4, 128).to(torch.bfloat16).to(dev)
    k = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(2, 4, 5, device=dev)
    out = torch.full((2, 5, 4, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    sdpa.prefill(q, k, k, causal=False, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_prefill_special_values(dev, oracle_mod):
    g = torch.Generator().manual_seed(5)
    B, Sq, Sk, Hq, Hkv, D = 1, 70, 150, 4, 2, 128
    q = torch.randn(B, Sq, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(torch.bfloat16)
    # scale = 0: uniform average of the visible values
    _prefill_case(dev, oracle_mod, q, k, v, causal=True, scale=0.0, what="scale=0")
    # constant V rows give that constant exactly (bf16-representable 0.75):
    # the row sum is over the fp32 probabilities, their bf16 roundings differ
    # from it by at most 2^-9 relative, 0.0015 at 0.75, under half a bf16 ulp
    vc = torch.full_like(v, 0.75)
    out = _prefill_case(dev, oracle_mod, q, k, vc, causal=True, scale=0.1, what="constant V")
    assert torch.equal(out.float().cpu(), torch.full((B, Sq, Hq, D), 0.75))
    # large logits: near one-hot rows, no overflow
    _prefill_case(dev, oracle_mod, (q.float() * 8).to(torch.bfloat16), k, v, causal=False, scale=1.0,
                  what="large logits", check_lse=False)


def test_prefill_deterministic(dev):
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w, q_len=200, kv_len=333)
    q, k, v = (t.to(dev) for t in (q, k, v))
    a = sdpa.prefill(q, k, v, causal=True)
    b = sdpa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------------ decode
def _decode_case(dev, oracle_mod, q, k, v, *, scale, num_splits=0, tol=TOL16, what=""):
    B, Hq, D = q.shape
    _say(f"decode {what} q={tuple(q.shape)} k={tuple(k.shape)} splits={num_splits}")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.full((B, Hq, v.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.decode(qd, kd, vd, scale=scale, out=out, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    ref = oracle_mod.sdpa(q.reshape(B, 1, Hq, D), k, v, scale=scale, causal=False)
    _compare(out, ref["out"][:, 0], tol, "out")
    got = lse.double().cpu().numpy()
    want = ref["lse"][:, :, 0]
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.abs(got[fin] - want[fin]).max(initial=0) <= _lse_tol(q.dtype)
    return out


@pytest.mark.parametrize("kv_set", [0, 1, 2, 3])
def test_splitkv_decode_bf16(dev, oracle_mod, kv_set):
    """The full decode workload, every row, on each of its four rotating K/V
    sets (the seeded recipe: seed + 100 * set)."""
    w = inputs.WORKLOADS["splitkv_decode_bf16"]
    q, k, v, _ = inputs.make_qkv(w, kv_set=kv_set)
    _decode_case(dev, oracle_mod, q.reshape(w.batch, w.head_q, w.d_qk), k, v, scale=w.scale,
                 what=f"{w.name} set {kv_set}")


DECODE_EDGE = [
    # B, Sk, Hq, Hkv, D, dtype, splits
    (1, 1, 4, 4, 128, torch.bfloat16, 0),
    (2, 31, 8, 2, 128, torch.float16, 0),
    (3, 100, 16, 1, 64, torch.bfloat16, 9),    # more splits than blocks: empty splits
    (2, 1000, 32, 8, 128, torch.bfloat16, 3),
    (1, 4097, 2, 1, 128, torch.bfloat16, 0),
    (4, 333, 12, 4, 64, torch.float16, 0),
    (3, 70, 6, 2, 128, torch.bfloat16, 0),     # 18 (batch, head) rows: a partly filled combine workgroup
    (1, 2000, 6, 3, 64, torch.float16, 40),    # more than 32 splits (looped combine), 6 rows
    (2, 1500, 64, 2, 128, torch.bfloat16, 0),  # 32 query heads per KV head: two 16-head tiles per KV head
    (3, 700, 20, 1, 64, torch.float16, 0),     # 20 per KV head: a full and a 4-head tile
    (1, 900, 160, 5, 128, torch.bfloat16, 3),  # 32 per KV head, 10 tasks: a partly filled workgroup
]


@pytest.mark.parametrize("case", DECODE_EDGE, ids=[f"B{c[0]}_k{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_s{c[6]}" for c in DECODE_EDGE])
def test_decode_edge_shapes(dev, oracle_mod, case):
    B, Sk, Hq, Hkv, D, dt, splits = case
    g = torch.Generator().manual_seed(Sk + 17 * Hq)
    q = torch.randn(B, Hq, D, generator=g).to(dt)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    v = torch.randn(B, Sk, Hkv, D, generator=g).to(dt)
    _decode_case(dev, oracle_mod, q, k, v, scale=1 / math.sqrt(D), num_splits=splits)


def test_decode_kv_len_zero(dev):
    q = torch.randn(2, 8, 128).to(torch.bfloat16).to(dev)
    k = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(2, 8, device=dev)
    out = torch.full((2, 8, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    sdpa.decode(q, k, k, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_binding_rejects_mismatched_device_tensors(dev):
    """Mismatched device tensors are refused by the binding before any launch
    (an fp8 K under bf16 Q, a short K batch or a small out / lse would
    otherwise be indexed past their ends)."""
    q = torch.zeros(2, 64, 8, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(2, 96, 2, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(2, 96, 2, 128, dtype=torch.bfloat16, device=dev)
    bad = [
        dict(k=k.to(torch.float8_e4m3fn)),
        dict(k=k[:1].contiguous(), v=v[:1].contiguous()),
        dict(v=v[:, :95].contiguous()),
        dict(out=torch.empty(2, 64, 8, 64, dtype=torch.bfloat16, device=dev)),
        dict(out=torch.empty(2, 64, 8, 128, dtype=torch.float16, device=dev)),
        dict(lse=torch.empty(2, 8, 63, dtype=torch.float32, device=dev)),
        dict(lse=torch.empty(2, 8, 64, dtype=torch.float16, device=dev)),
    ]
    for case in bad:
        args = dict(q=q, k=k, v=v)
        args.update({n: t for n, t in case.items() if n in ("k", "v")})
        kw = {n: t for n, t in case.items() if n in ("out", "lse")}
        with pytest.raises(ValueError):
            sdpa.prefill(args["q"], args["k"], args["v"], causal=True, **kw)
    qd = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        sdpa.decode(qd, k.to(torch.float16), v)
    with pytest.raises(ValueError):
        sdpa.decode(qd, k, v, out=torch.empty(2, 8, 64, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        sdpa.decode(qd, k, v, lse=torch.empty(2, 4, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
