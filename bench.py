"""Benchmark of the fused SDPA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one call of the hot path on its workload:
  * headline: causal GQA bf16 prefill (batch 1, 32 query / 8 KV heads,
    q_len 512, kv_len 1024, head dim 128) -- `value` is its attention
    TFLOP/s over algorithmic FLOP (2*(D+Dv) per visible query-key pair);
  * "decode": two-phase split-KV decode (batch 16, 32/8 heads, kv_len 8192,
    head dim 128, bf16), K/V rotated over 4 buffer sets between calls so the
    cache cannot serve them -- achieved HBM GB/s over algorithmic bytes
    (Q + K + V read once, O written once).
Inputs are resident in HBM before the timed region.  Each timed region is
W untimed calls, synchronize, K back-to-back calls bracketed by HIP events on
the stream the kernels run on, synchronize.  Rank 0 prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2    # dense fp8
PEAK_HBM_GBS = 8000.0       # HBM3E


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_flash_sdpa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(profile_name, src_names):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when the summary is missing or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != _src_hash(*src_names):
        return None
    return float(t.group(1))


def _time(fn, steps, warmup, stream):
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms per call


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the attention path "
              "shards by heads with no communication, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sdpa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)

    # ---------------- headline: causal GQA bf16 prefill ----------------
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty(w.batch, w.q_len, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    ms = _time(lambda i: sdpa.prefill(qd, kd, vd, scale=w.scale, causal=True, out=out), args.steps, args.warmup,
               stream)
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    plan = sdpa.plan(sdpa.make_problem(batch=w.batch, q_len=w.q_len, kv_len=w.kv_len, head_q=w.head_q,
                                       head_kv=w.head_kv, d_qk=w.d_qk, d_v=w.d_v, in_dtype=sdpa.BF16,
                                       out_dtype=sdpa.BF16, causal=True, scale=w.scale))

    # sampled parity of the timed output against the oracle
    import oracle

    rows = np.array([(0, i, h) for i in (0, 1, 255, 511) for h in (0, 13, 31)], dtype=np.int64)
    ref = oracle.sdpa(q, k, v, scale=w.scale, causal=True, rows=rows, want_lse=False)["out"]
    got = out.cpu()[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    prefill_err = float(np.abs(got - ref).max())
    prefill_nan = int(np.isnan(got).sum())

    # ---------------- split-KV decode, 4 rotating K/V sets ----------------
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    dq, dk0, dv0, _ = inputs.make_qkv(dw)
    dqd = dq.reshape(dw.batch, dw.head_q, dw.d_qk).to(dev)
    sets = [(dk0.to(dev), dv0.to(dev))]
    for s in range(1, dw.kv_sets):
        g = torch.Generator(device=dev).manual_seed(dw.seed + 100 * s)
        sets.append(tuple(torch.randn(t.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                          for t in (dk0, dv0)))
    dout = torch.empty(dw.batch, dw.head_q, dw.d_v, dtype=torch.bfloat16, device=dev)
    ws = sdpa.decode_workspace(dqd, sets[0][0], sets[0][1])
    dms = _time(lambda i: sdpa.decode(dqd, sets[i % len(sets)][0], sets[i % len(sets)][1], scale=dw.scale,
                                      out=dout, workspace=ws),
                args.decode_steps, args.warmup, stream)
    dbytes = dw.bytes_moved()
    dgbs = dbytes / (dms * 1e-3) / 1e9
    dplan = sdpa.plan(sdpa.make_problem(batch=dw.batch, q_len=1, kv_len=dw.kv_len, head_q=dw.head_q,
                                        head_kv=dw.head_kv, d_qk=dw.d_qk, d_v=dw.d_v, in_dtype=sdpa.BF16,
                                        out_dtype=sdpa.BF16, causal=False, scale=dw.scale),
                      decode=True, num_cus=props.multi_processor_count)
    sdpa.decode(dqd, sets[0][0], sets[0][1], scale=dw.scale, out=dout, workspace=ws)
    torch.cuda.synchronize()
    drows = np.array([(b, 0, h) for b in (0, 7, 15) for h in (0, 17, 31)], dtype=np.int64)
    dref = oracle.sdpa(dq, dk0, dv0, scale=dw.scale, causal=False, rows=drows, want_lse=False)["out"]
    dgot = dout.cpu()[drows[:, 0], drows[:, 2]].double().numpy()
    decode_err = float(np.abs(dgot - dref).max())

    # ---------------- other prefill workloads (context lines) ----------------
    extra = {}
    for name in ("single_head_f16_128", "unaligned_full_bf16", "tiny_causal_bf16", "mla_fp8_causal_prefill"):
        xw = inputs.WORKLOADS[name]
        xq, xk, xv, xds = inputs.make_qkv(xw)
        xq, xk, xv = (t.to(dev) for t in (xq, xk, xv))
        odt = torch.bfloat16 if xw.out_dtype == "bf16" else torch.float16
        xo = torch.empty(xw.batch, xw.q_len, xw.head_q, xw.d_v, dtype=odt, device=dev)
        n = 100 if xw.flops() < 1e9 else max(args.steps // 4, 1)
        xms = _time(lambda i: sdpa.prefill(xq, xk, xv, scale=xw.scale, causal=xw.causal, out=xo, descale=xds),
                    n, args.warmup, stream)
        xt = xw.flops() / (xms * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if xw.dtype == "fp8_e4m3" else PEAK_BF16_TFLOPS
        extra[name] = {"value": round(xt, 3), "unit": "TFLOP/s", "ms_per_call": round(xms, 6), "steps": n,
                       "algorithmic_gflop": round(xw.flops() / 1e9, 4), "peak": peak,
                       "frac_of_peak": round(xt / peak, 5)}
        del xq, xk, xv, xo
    # launch floor: a one-element device op timed the same way
    one = torch.zeros(1, device=dev)
    floor_ms = _time(lambda i: one.add_(1.0), args.steps, args.warmup, stream)

    # ---------------- CPU baseline: the oracle on the host cores ----------------
    cpu = None
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        os.environ["OMP_NUM_THREADS"] = str(threads)
        t0 = time.perf_counter()
        oracle.sdpa(q, k, v, scale=w.scale, causal=True, want_lse=False, threads=threads)
        sec = time.perf_counter() - t0
        cpu = {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"whole causal GQA prefill workload ({w.batch * w.q_len * w.head_q} rows, "
                         f"{flops / 1e9:.2f} GFLOP) in {sec:.2f} s, fp64, {_cpu_model()}"}

    traffic = _traffic("prefill_gqa_causal_bf16_counters.txt", ["prefill.hip", "sdpa_device.h"])
    dtraffic = _traffic("decode_splitkv_bf16_counters.txt", ["decode.hip", "sdpa_device.h"])
    line = {
        "metric": "attention TFLOP/s (causal GQA bf16 prefill) + decode achieved HBM GB/s, 1 GPU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": w.name, "batch": w.batch, "head_q": w.head_q, "head_kv": w.head_kv,
                   "q_len": w.q_len, "kv_len": w.kv_len, "d_qk": w.d_qk, "d_v": w.d_v, "causal": True,
                   "algorithmic_gflop": round(flops / 1e9, 4), "grid": plan.num_groups},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 5), "traffic": traffic},
        "cpu_baseline": cpu,
        "parity": {"max_abs_err": prefill_err, "nan": prefill_nan, "sampled_rows": int(len(rows))},
        "decode": {
            "workload": dw.name, "value": round(dgbs, 2), "unit": "GB/s", "ms_per_call": round(dms, 6),
            "steps": args.decode_steps, "kv_sets": dw.kv_sets, "num_splits": dplan.num_splits,
            "algorithmic_bytes": dbytes,
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dgbs / PEAK_HBM_GBS, 5), "traffic": dtraffic},
            "parity": {"max_abs_err": decode_err},
        },
        "other_workloads": extra,
        "launch_floor_us": round(floor_ms * 1e3, 3),
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
