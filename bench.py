"""Benchmark of the fused SDPA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --counters-pass              # short run for rocprofv3 --pmc
    python bench.py --summarize-trace DIR        # kernel-trace CSV -> profiles/
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR
    python bench.py --summarize-sq DIR           # SQ counter run -> profiles/

One step = one call of the hot path on its workload:
  * headline: causal GQA bf16 prefill (batch 1, 32 query / 8 KV heads,
    q_len 512, kv_len 1024, head dim 128) -- `value` is its attention
    TFLOP/s over algorithmic FLOP (2*(D+Dv) per visible query-key pair);
  * "decode": two-phase split-KV decode (batch 16, 32/8 heads, kv_len 8192,
    head dim 128, bf16), K/V rotated over 4 buffer sets between calls so the
    cache cannot serve them -- achieved HBM GB/s over algorithmic bytes
    (Q + K + V read once, O written once).
Inputs are resident in HBM before the timed region.  The calls go through the
Python binding and the C ABI; a chunk of C consecutive calls (the largest
divisor of K that is a multiple of the input-rotation period, at most 200) is
captured once into a HIP graph (the library allocates and synchronizes
nothing, so its launches capture as they are).  At least one untimed replay
(and at least W untimed calls), then K/C replays bracketed by HIP events on
the stream the kernels run on.  The prefill step is a single kernel, so its
time per step is that kernel's launch-to-launch period back to back, an upper
bound of its average duration.  The same K calls issued one by one from Python are timed too
("eager", host-bound for small workloads).  Rank 0 prints ONE JSON line.
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


def _progress(msg):
    """A progress line on stderr (the JSON line stays alone on stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _cpu_line(value, unit, cores, sample):
    """The oracle as it stands, timed on the host beside a GPU leg."""
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}


def _time(fn, steps, warmup, stream):
    """Eager: K back-to-back calls from Python, after W warmup calls."""
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


def _graph_chunk(steps, period, cap=200):
    """Calls per captured graph: the largest divisor of `steps` that is a
    multiple of `period` (rotating inputs keep their order) and at most `cap`
    (`steps` itself is rounded up to a multiple of `period` first)."""
    steps = -(-steps // period) * period
    best = period
    for c in range(period, min(steps, cap) + 1, period):
        if steps % c == 0:
            best = c
    return steps, best


def _graph_time(fn, steps, warmup, period=1):
    """K calls as replays of one captured chunk of C calls (C divides K and is
    a multiple of `period`); at least one untimed replay (and at least W
    untimed calls) first, then K/C replays between HIP events on the launch
    stream.  Returns ms per call."""
    import torch

    steps, c = _graph_chunk(steps, period)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(c):
            fn(i)
    for _ in range(max(1, -(-warmup // c))):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps // c):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


# timed calls of each secondary leg at least (independent of --steps)
MIN_LEG_CALLS = 20


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _problem(sdpa, w):
    code = {"f16": sdpa.F16, "bf16": sdpa.BF16, "fp8_e4m3": sdpa.FP8_E4M3}
    return sdpa.make_problem(batch=w.batch, q_len=1 if w.decode else w.q_len, kv_len=w.kv_len, head_q=w.head_q,
                             head_kv=w.head_kv, d_qk=w.d_qk, d_v=w.d_v, in_dtype=code[w.dtype],
                             out_dtype=code[w.out_dtype], causal=w.causal, scale=w.scale)


def _kernels_of(sdpa, w, num_cus=256, paged=False, cached=False):
    """(kernel name, grid size in work-items) of each launch one call of
    workload `w` makes, from the host planner (`paged`: decode through a page
    table; `cached`: prefill over a cached prefix, `w.kv_len` counting cache
    and new keys)."""
    p = sdpa.plan(_problem(sdpa, w), decode=w.decode, num_cus=num_cus)
    t = {"f16": "F16", "bf16": "Bf16"}.get(w.dtype)
    c = "true" if w.causal else "false"
    if w.decode:
        return [(f"decode_split_kernel<sdpa::{t}, {w.d_qk}, {w.d_v}, {'true' if paged else 'false'}>",
                 p.num_groups * p.waves_per_group * 64),
                (f"decode_combine_kernel<sdpa::{t}, {w.d_v}>", p.combine_groups * 256)]
    if w.dtype == "fp8_e4m3":
        return [(f"prefill_fp8_kernel<{c}>", p.num_groups * p.waves_per_group * 64)]
    if 12 <= p.kernel <= 15 or 24 <= p.kernel <= 27:   # the two-waves-per-SIMD 32-row kernel
        shape = "4, 1, 64" if p.kernel <= 15 else "8, 4, 32"   # waves, key ranges, keys per block
        return [(f"prefill_o2_kernel<sdpa::{t}, {w.d_qk}, {w.d_v}, {c}, {shape}, {'true' if cached else 'false'}, false>",
                 p.num_groups * p.waves_per_group * 64)]
    if cached:
        # the cached form whose fills take a scalar base: cache length and key
        # count multiples of the 512 / D rows one fill instruction covers
        rstep = 512 // w.d_qk
        align = "true" if CACHED_LEN % rstep == 0 and w.kv_len % rstep == 0 else "false"
        return [(f"prefill_kernel<sdpa::{t}, {w.d_qk}, {w.d_v}, {c}, {p.num_splits}, true, {align}, false>",
                 p.num_groups * p.waves_per_group * 64)]
    if p.kv_splits > 1:  # keys split across workgroups: the partials' combine follows
        return [(f"prefill_kernel<sdpa::{t}, {w.d_qk}, {w.d_v}, {c}, {p.num_splits}, false, false, true>",
                 p.num_groups * p.waves_per_group * 64),
                (f"decode_combine_kernel<sdpa::{t}, {w.d_v}>", p.combine_groups * 256)]
    return [(f"prefill_kernel<sdpa::{t}, {w.d_qk}, {w.d_v}, {c}, {p.num_splits}, false, false, false>",
             p.num_groups * p.waves_per_group * 64)]


# kernel-source files whose text decides each profiled kernel's code
_SOURCES = {"prefill": ["prefill.hip", "prefill_kernel.h", "prefill_o2.hip", "prefill_o2_kernel.h",
                        "sdpa_device.h", "lds_layout.h", "sdpa_internal.h", "sdpa_bounds.h"],
            "decode": ["decode.hip", "sdpa_device.h", "lds_layout.h", "sdpa_internal.h"],
            "fp8": ["prefill_fp8.hip", "sdpa_device.h", "lds_layout.h", "sdpa_internal.h", "sdpa_bounds.h"],
            "masked": ["prefill_o2.hip", "prefill_o2_kernel.h", "sdpa_device.h", "lds_layout.h", "sdpa_internal.h",
                       "sdpa_bounds.h"],
            "mask": ["mask.hip", "sdpa_device.h", "sdpa_internal.h"],
            "split": ["prefill_split.hip", "prefill_kernel.h", "decode.hip", "sdpa_device.h", "lds_layout.h",
                      "sdpa_internal.h", "sdpa_bounds.h"]}
SPLIT_COUNTERS = "prefill_split_chunk16_over8192_bf16_counters.txt"
def _cached_chunk():
    from attention_flash_sdpa_amd import inputs

    # a 512-query chunk over 3584 cached keys (4096 keys in all); q_len and
    # kv_len as the planner sees them
    return inputs.Workload("cached_prefill_chunk512_over3584_bf16", 1, 32, 8, 512, 4096, 128, 128, "bf16", "bf16",
                           True, 1006)


CACHED_CHUNK = _cached_chunk()


def _split_chunk():
    from attention_flash_sdpa_amd import inputs

    # a 16-query chunk over 8192 keys: too few query tiles to fill the GPU,
    # so the planner splits each tile's keys across workgroups
    return inputs.Workload("short_chunk16_over8192_bf16", 1, 32, 8, 16, 8192, 128, 128, "bf16", "bf16", True, 1009,
                           kv_sets=8)


SPLIT_CHUNK = _split_chunk()
MASK_SHAPE = (16, 4096, 4096)  # bool mask elements converted per call


def _masked_workload():
    from attention_flash_sdpa_amd import inputs

    return inputs.Workload("masked_prefill_bias_2048_bf16", 1, 32, 8, 2048, 2048, 128, 128, "bf16", "bf16", False,
                           1008)


MASKED = _masked_workload()
# the masked prefill runs the two-waves-per-SIMD kernel with the bias form on
MASKED_KERNEL = "prefill_o2_kernel<sdpa::Bf16, 128, 128, false, 4, 1, 64, false, true>"
CACHED_LEN = 3584

_PROFILED = {"gqa_causal_prefill_bf16": "prefill_gqa_causal_bf16", "splitkv_decode_bf16": "decode_splitkv_bf16"}
PAGED_PROFILED = (64, 16)  # page sizes of the paged decode in the counters pass, in this order


def _counters_pass():
    """Short run for `rocprofv3 --pmc`: a plain 256 MiB device copy (the
    calibration of the byte counters), then 5 calls each of the causal GQA
    prefill and of the split-KV decode (rotating K/V sets), then 6 mask
    conversions (two alternating buffer sets)."""
    import torch

    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    qd, kd, vd = (t.to(dev) for t in inputs.make_qkv(w)[:3])
    out = torch.empty(w.batch, w.q_len, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    dq, dk0, dv0, _ = inputs.make_qkv(dw)
    dqd = dq.reshape(dw.batch, dw.head_q, dw.d_qk).to(dev)
    sets = [(dk0.to(dev), dv0.to(dev))] + [
        (torch.empty_like(dk0, device=dev).normal_(), torch.empty_like(dv0, device=dev).normal_())
        for _ in range(1, dw.kv_sets)]
    dout = torch.empty(dw.batch, dw.head_q, dw.d_v, dtype=torch.bfloat16, device=dev)
    ws = sdpa.decode_workspace(dqd, sets[0][0], sets[0][1])
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(5):
        sdpa.prefill(qd, kd, vd, scale=w.scale, causal=True, out=out)
    torch.cuda.synchronize()
    for i in range(4 * 5):
        sdpa.decode(dqd, sets[i % 4][0], sets[i % 4][1], scale=dw.scale, out=dout, workspace=ws)
    torch.cuda.synchronize()
    del sets
    # the paged decode over set 0: 5 calls in 64-key pages, then 5 in 16-key
    # pages (its 537 MB of K/V exceed the last-level cache, so every call
    # reads from HBM)
    full = torch.full((dw.batch,), dw.kv_len, dtype=torch.int32, device=dev)
    for ps in PAGED_PROFILED:
        kp, vp, table = (t.to(dev) for t in inputs.paginate(dk0, dv0, ps, seed=dw.seed + 1))
        for _ in range(5):
            sdpa.decode_paged(dqd, kp, vp, page_table=table, seq_lens=full, scale=dw.scale, out=dout, workspace=ws)
        torch.cuda.synchronize()
        del kp, vp, table
    msets = [(torch.rand(MASK_SHAPE, device=dev) < 0.5, torch.empty(MASK_SHAPE, dtype=torch.bfloat16, device=dev))
             for _ in range(2)]
    for i in range(6):
        sdpa.mask_convert(msets[i % 2][0], out=msets[i % 2][1])
    torch.cuda.synchronize()
    del msets
    # the other profiled prefills: 3 calls each
    for name in ("unaligned_full_bf16", "mla_fp8_causal_prefill"):
        xw = inputs.WORKLOADS[name]
        xq, xk, xv, xds = inputs.make_qkv(xw)
        xq, xk, xv = (t.to(dev) for t in (xq, xk, xv))
        for _ in range(3):
            sdpa.prefill(xq, xk, xv, scale=xw.scale, causal=xw.causal, descale=xds)
        torch.cuda.synchronize()
        del xq, xk, xv
    cw = CACHED_CHUNK
    g = torch.Generator().manual_seed(cw.seed)
    new = cw.kv_len - CACHED_LEN
    cq = torch.randn(1, cw.q_len, cw.head_q, cw.d_qk, generator=g).to(torch.bfloat16).to(dev)
    ckc, cvc, ck, cv = (torch.randn(1, n, cw.head_kv, cw.d_qk, generator=g).to(torch.bfloat16).to(dev)
                        for n in (CACHED_LEN, CACHED_LEN, new, new))
    for _ in range(3):
        sdpa.prefill_cached(cq, ckc, cvc, ck, cv, cache_len=CACHED_LEN, causal=True, scale=cw.scale)
    torch.cuda.synchronize()
    mq, mk, mv, mbias = _masked_inputs(dev)
    for _ in range(3):
        sdpa.prefill_masked(mq, mk, mv, mbias, scale=MASKED.scale)
    torch.cuda.synchronize()
    del mq, mk, mv, mbias
    # the split prefill leg: one call per rotating K/V set (past the
    # last-level cache, so every call reads its keys from HBM)
    sw = SPLIT_CHUNK
    g = torch.Generator().manual_seed(sw.seed)
    sq = torch.randn(sw.batch, sw.q_len, sw.head_q, sw.d_qk, generator=g).to(torch.bfloat16).to(dev)
    s_sets = [tuple(torch.randn(sw.batch, sw.kv_len, sw.head_kv, sw.d_qk, generator=g).to(torch.bfloat16).to(dev)
                    for _ in range(2)) for _ in range(sw.kv_sets)]
    sws = torch.empty(sdpa.prefill_workspace_bytes(sq, *s_sets[0], causal=True), dtype=torch.uint8, device=dev)
    for kk, vv in s_sets:
        sdpa.prefill(sq, kk, vv, causal=True, scale=sw.scale, workspace=sws)
    torch.cuda.synchronize()
    print(f"counters pass done: copy {src.numel()} B x3, prefill x5, decode x20, paged decode x5 per page size, "
          f"mask conversion x6, unaligned / fp8 / cached / masked prefill x3 each, split prefill x{sw.kv_sets}",
          flush=True)


def _masked_inputs(dev):
    """The masked-prefill leg's inputs: seeded Q, K, V and a per-head linear
    distance bias [1, Hq, Sq, Sk] (slopes 2^(-h/4)), on the device."""
    import torch

    xw = MASKED
    g = torch.Generator().manual_seed(xw.seed)
    mq = torch.randn(1, xw.q_len, xw.head_q, xw.d_qk, generator=g).to(torch.bfloat16)
    mk = torch.randn(1, xw.kv_len, xw.head_kv, xw.d_qk, generator=g).to(torch.bfloat16)
    mv = torch.randn(1, xw.kv_len, xw.head_kv, xw.d_v, generator=g).to(torch.bfloat16)
    ii = torch.arange(xw.q_len, device=dev)[:, None]
    jj = torch.arange(xw.kv_len, device=dev)[None, :]
    slope = 2.0 ** (-torch.arange(1, xw.head_q + 1, device=dev) / 4.0)
    mbias = (-(slope[:, None, None] * (ii - jj).abs()[None])).to(torch.bfloat16)[None].contiguous()
    return mq.to(dev), mk.to(dev), mv.to(dev), mbias


# SQ counters of one --pmc pass (at most 8 SQ and 2 GRBM counters per pass)
SQ_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU",
               "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "GRBM_GUI_ACTIVE")


def _sq_profiles():
    """(profile stem, kernel-name fragment, grid work-items or None, source
    files, workload label) of every kernel the SQ summary covers."""
    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    out = []
    for wname in ("gqa_causal_prefill_bf16", "unaligned_full_bf16", "mla_fp8_causal_prefill", "splitkv_decode_bf16"):
        w = inputs.WORKLOADS[wname]
        for kname, grid in _kernels_of(sdpa, w):
            fam = kname.split("<")[0]
            src = _SOURCES["decode"] if w.decode else (_SOURCES["fp8"] if w.dtype == "fp8_e4m3" else
                                                       _SOURCES["prefill"])
            out.append((f"{fam}_{wname}", kname, grid, src, wname))
    for kname, grid in _kernels_of(sdpa, CACHED_CHUNK, cached=True):
        out.append((f"{kname.split('<')[0]}_{CACHED_CHUNK.name}", kname, grid, _SOURCES["prefill"], CACHED_CHUNK.name))
    out.append((f"prefill_o2_kernel_{MASKED.name}", MASKED_KERNEL, None, _SOURCES["masked"], MASKED.name))
    return out


def _summarize_sq(d):
    """Per-kernel SQ counter summaries (MFMA busy, instruction mix, LDS bank
    conflicts) from one `rocprofv3 --pmc <SQ_COUNTERS>` run of the counters
    pass, written to profiles/<kernel>_<workload>_sq_counters.txt."""
    import statistics

    rows = _read_csv(os.path.join(d, "run_counter_collection.csv"))
    for stem, kname, grid, src, wname in _sq_profiles():
        per = {}
        for r in rows:
            if kname in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid):
                per.setdefault(r["Counter_Name"], {}).setdefault(int(r["Dispatch_Id"]), 0.0)
                per[r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        if not per:
            continue
        avg = {c: statistics.mean(v.values()) for c, v in per.items()}
        n = max(len(v) for v in per.values())
        out = os.path.join(ROOT, "profiles", f"{stem}_sq_counters.txt")
        with open(out, "w") as f:
            f.write(f"kernel: {kname}\nworkload: {wname}\n")
            f.write(f"command:\n  rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d {d} -o run "
                    f"-- python3 bench.py --counters-pass\n  python3 bench.py --summarize-sq {d}\n")
            f.write(f"dispatches: {n}\nper dispatch (mean):\n")
            for c in SQ_COUNTERS:
                if c in avg:
                    f.write(f"  {c}: {avg[c]:.0f}\n")
            mf, valu = avg.get("SQ_INSTS_MFMA"), avg.get("SQ_INSTS_VALU")
            busy, cu = avg.get("SQ_VALU_MFMA_BUSY_CYCLES"), avg.get("SQ_BUSY_CU_CYCLES")
            if mf and valu:
                f.write(f"non-MFMA VALU instructions per MFMA: {(valu - mf) / mf:.2f}\n")
            if busy and cu:
                # busy cycles are counted per SIMD (32 per 32x32x16 MFMA), CU-busy
                # cycles per CU: four SIMDs per CU
                f.write(f"MFMA busy share of SIMD cycles while the CUs are busy, "
                        f"SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES): {busy / (4 * cu):.3f}\n")
            if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_INSTS_LDS" in avg and avg["SQ_INSTS_LDS"]:
                f.write(f"LDS bank-conflict cycles per LDS instruction: "
                        f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_INSTS_LDS']:.3f}\n")
            f.write(f"source_sha256: {_src_hash(*src)}\n")
        print("wrote", out)


def _read_csv(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _summarize_trace(d):
    """Per-workload kernel-duration summaries from a `rocprofv3 --kernel-trace
    --stats` run of bench.py, written to profiles/<kernel>_<workload>_trace.txt."""
    import statistics

    import numpy as np

    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    rows = _read_csv(os.path.join(d, "run_kernel_trace.csv"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # a prefill split across workgroups launches its kernel and then the
    # combine, whose name and grid are the decode's: told apart by the launch
    # beside it (one stream, in order)
    for i, r in enumerate(rows):
        r["_next"] = rows[i + 1]["Kernel_Name"] if i + 1 < len(rows) else ""
        r["_prev"] = rows[i - 1]["Kernel_Name"] if i > 0 else ""
    cmd = open(os.path.join(d, "command.txt")).read().strip() if os.path.exists(os.path.join(d, "command.txt")) \
        else "(command not recorded)"
    todo = [(wname, w, False) for wname, w in inputs.WORKLOADS.items()]
    todo.append(("splitkv_decode_bf16_paged_16_and_64", inputs.WORKLOADS["splitkv_decode_bf16"], True))
    todo.append((CACHED_CHUNK.name, CACHED_CHUNK, "cached"))
    todo.append((SPLIT_CHUNK.name, SPLIT_CHUNK, False))
    todo.append(("mask_convert_16x4096x4096", None, "mask"))
    todo.append((MASKED.name, MASKED, "masked"))
    for wname, w, paged in todo:
        if paged == "mask":
            kernels = [("mask_convert_kernel", None)]
        elif paged == "masked":
            kernels = [(MASKED_KERNEL, None)]
        else:
            kernels = _kernels_of(sdpa, w, paged=paged is True, cached=paged == "cached")
        split = w is not None and not w.decode and paged is False and \
            sdpa.plan(_problem(sdpa, w), num_cus=256).kv_splits > 1
        for kname, grid in kernels:
            if paged is True and "true>" not in kname:
                continue  # the combine kernel is the dense one

            def hit(r):
                if kname not in r["Kernel_Name"] or (grid is not None and int(r["Grid_Size_X"]) != grid):
                    return False
                if kname.startswith("prefill_kernel<"):
                    return ("decode_combine_kernel" in r["_next"]) == split
                if kname.startswith("decode_combine_kernel<"):
                    return ("prefill_kernel<" in r["_prev"]) == split
                return True

            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if hit(r)]
            if not durs:
                continue
            r0 = next(r for r in rows if hit(r))
            grid = int(r0["Grid_Size_X"])
            fam = kname.split("<")[0]
            out = os.path.join(ROOT, "profiles", f"{fam}_{wname}_trace.txt")
            byte_bound = w is None or w.decode or split
            alg = 3 * int(np.prod(MASK_SHAPE)) if w is None else (w.bytes_moved() if byte_bound else w.flops())
            with open(out, "w") as f:
                f.write(f"kernel: {r0['Kernel_Name']}\nworkload: {wname}\n")
                f.write(f"command: {cmd}\n")
                f.write(f"grid work-items: {grid}  workgroup: {r0['Workgroup_Size_X']}  lds_bytes: "
                        f"{r0['LDS_Block_Size']}  scratch: {r0['Scratch_Size']}  vgpr: {r0['VGPR_Count']}  "
                        f"agpr: {r0['Accum_VGPR_Count']}  sgpr: {r0['SGPR_Count']}\n")
                f.write(f"dispatches: {len(durs)}\n")
                f.write(f"avg_us: {statistics.mean(durs):.3f}\nmedian_us: {statistics.median(durs):.3f}\n"
                        f"min_us: {min(durs):.3f}\nmax_us: {max(durs):.3f}\n")
                if w is None:
                    f.write(f"algorithmic bytes per call (mask read + additive mask written): {alg}\n"
                            f"GB/s at median: {alg / statistics.median(durs) / 1e3:.1f}\n")
                elif byte_bound:
                    f.write(f"algorithmic bytes per call (Q+K+V+O): {alg}\n")
                    if split:
                        f.write("the call is this kernel and the combine of its partials\n")
                else:
                    med = statistics.median(durs)
                    f.write(f"algorithmic flop per call: {alg}\nTFLOP/s at median: {alg / med / 1e6:.1f}\n")
            print("wrote", out)


def _summarize_counters(fetch_dir, write_dir):
    """HBM bytes per launch from two `rocprofv3 --pmc` runs of the counters
    pass (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter
    reads for the 256 MiB device copy, written to profiles/*_counters.txt."""
    import statistics

    import numpy as np

    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    copy_bytes = 256 << 20
    res = {}
    mres = {}  # mask conversion: (mean KiB per dispatch, dispatches)
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv")) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        first_sdpa = min(int(r["Dispatch_Id"]) for r in rows if "sdpa::" in r["Kernel_Name"])
        copies = [r for r in rows if "copy" in r["Kernel_Name"].lower() and int(r["Dispatch_Id"]) < first_sdpa][-3:]
        kib_copy = statistics.mean(float(r["Counter_Value"]) for r in copies)
        factor = copy_bytes / (kib_copy * 1024.0)
        per = {}
        for wname in _PROFILED:
            w = inputs.WORKLOADS[wname]
            for kname, grid in _kernels_of(sdpa, w):
                vals = [float(r["Counter_Value"]) for r in rows
                        if kname in r["Kernel_Name"] and int(r["Grid_Size"]) == grid]
                per[(wname, kname)] = (statistics.mean(vals), len(vals))
        res[counter] = (kib_copy, factor, per, copies[0]["Kernel_Name"])
        mvals = [float(r["Counter_Value"]) for r in rows if "mask_convert_kernel" in r["Kernel_Name"]]
        if mvals:
            mres[counter] = (statistics.mean(mvals), len(mvals))
    for wname, stem in _PROFILED.items():
        w = inputs.WORKLOADS[wname]
        kind = "decode" if w.decode else "prefill"
        out = os.path.join(ROOT, "profiles", f"{stem}_counters.txt")
        total = 0.0
        with open(out, "w") as f:
            f.write(f"workload: {wname}\n")
            f.write(f"commands:\n  rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run "
                    f"-- python3 bench.py --counters-pass\n  rocprofv3 --pmc WRITE_SIZE --output-format csv "
                    f"-d {write_dir} -o run -- python3 bench.py --counters-pass\n"
                    f"  python3 bench.py --summarize-counters {fetch_dir} {write_dir}\n")
            for counter in ("FETCH_SIZE", "WRITE_SIZE"):
                kib_copy, factor, per, cname = res[counter]
                f.write(f"{counter}: calibration copy of {copy_bytes} B ({cname}) reads {kib_copy:.1f} KiB "
                        f"-> scale factor {factor:.4f}\n")
                for (wn, kname), (kib, n) in per.items():
                    if wn != wname:
                        continue
                    b = kib * 1024.0 * factor
                    total += b
                    f.write(f"  {kname}: {kib:.1f} KiB/dispatch over {n} dispatches -> {b:.0f} B\n")
            alg = w.bytes_moved()
            f.write(f"algorithmic bytes per call (Q+K+V+O once): {alg}\n")
            f.write(f"hbm_bytes_per_launch: {total:.0f}\n")
            f.write(f"ratio to algorithmic: {total / alg:.3f}\n")
            f.write(f"source_sha256: {_src_hash(*_SOURCES[kind])}\n")
        print("wrote", out)
    # paged decode: its split-kernel dispatches in order (5 per page size),
    # each with the combine dispatch that follows it
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    ptot = {ps: 0.0 for ps in PAGED_PROFILED}
    plines = {ps: [] for ps in PAGED_PROFILED}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        kib_copy, factor, _, cname = res[counter]
        rows = {int(r["Dispatch_Id"]): r for r in _read_csv(os.path.join(d, "run_counter_collection.csv"))
                if r["Counter_Name"] == counter}
        split_ids = sorted(i for i, r in rows.items()
                           if "decode_split_kernel" in r["Kernel_Name"] and "true>" in r["Kernel_Name"])
        for k, ps in enumerate(PAGED_PROFILED):
            ids = split_ids[5 * k:5 * k + 5]
            if len(ids) < 5:
                continue
            sk = statistics.mean(float(rows[i]["Counter_Value"]) for i in ids)
            ck = statistics.mean(float(rows[i + 1]["Counter_Value"]) for i in ids
                                 if i + 1 in rows and "decode_combine_kernel" in rows[i + 1]["Kernel_Name"])
            b = (sk + ck) * 1024.0 * factor
            ptot[ps] += b
            plines[ps].append(f"{counter}: scale factor {factor:.4f} ({cname}); paged split kernel {sk:.1f} KiB + "
                              f"combine {ck:.1f} KiB per call over {len(ids)} calls -> {b:.0f} B\n")
    for ps in PAGED_PROFILED:
        if len(plines[ps]) != 2:
            continue
        out = os.path.join(ROOT, "profiles", f"decode_paged{ps}_splitkv_bf16_counters.txt")
        alg = dw.bytes_moved() + (dw.kv_len // ps) * dw.batch * 4 + dw.batch * 4
        with open(out, "w") as f:
            f.write(f"workload: splitkv_decode_bf16 in {ps}-key pages (shuffled physical order, every sequence full)\n")
            f.write("commands: as for decode_splitkv_bf16_counters.txt (the counters pass runs 5 paged calls per "
                    "page size after the dense decode)\n")
            for line in plines[ps]:
                f.write(line)
            f.write(f"algorithmic bytes per call (Q+K+V+O once, page table, lengths): {alg}\n")
            f.write(f"hbm_bytes_per_launch: {ptot[ps]:.0f}\n")
            f.write(f"ratio to algorithmic: {ptot[ps] / alg:.3f}\n")
            f.write(f"source_sha256: {_src_hash(*_SOURCES['decode'])}\n")
        print("wrote", out)
    # split prefill: each split-kernel dispatch with the combine dispatch that
    # follows it (the combine's name and grid are the decode's)
    sw = SPLIT_CHUNK
    skname = _kernels_of(sdpa, sw)[0][0]
    stot, slines = 0.0, []
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        kib_copy, factor, _, cname = res[counter]
        rows = {int(r["Dispatch_Id"]): r for r in _read_csv(os.path.join(d, "run_counter_collection.csv"))
                if r["Counter_Name"] == counter}
        ids = sorted(i for i, r in rows.items() if skname in r["Kernel_Name"])
        cids = [i for i in ids if i + 1 in rows and "decode_combine_kernel" in rows[i + 1]["Kernel_Name"]]
        if not ids or len(cids) != len(ids):
            continue
        sk = statistics.mean(float(rows[i]["Counter_Value"]) for i in ids)
        ck = statistics.mean(float(rows[i + 1]["Counter_Value"]) for i in ids)
        b = (sk + ck) * 1024.0 * factor
        stot += b
        slines.append(f"{counter}: scale factor {factor:.4f} ({cname}); {skname} {sk:.1f} KiB + combine "
                      f"{ck:.1f} KiB per call over {len(ids)} calls -> {b:.0f} B\n")
    if len(slines) == 2:
        out = os.path.join(ROOT, "profiles", SPLIT_COUNTERS)
        alg = sw.bytes_moved()
        with open(out, "w") as f:
            f.write(f"workload: {sw.name} ({sw.q_len} queries over {sw.kv_len} keys, {sw.head_q}/{sw.head_kv} heads, "
                    f"one call per rotating K/V set)\n")
            f.write("commands: as for prefill_gqa_causal_bf16_counters.txt (the counters pass ends with the split "
                    "prefill calls)\n")
            for line in slines:
                f.write(line)
            f.write(f"algorithmic bytes per call (Q+K+V+O once): {alg}\n")
            f.write(f"hbm_bytes_per_launch: {stot:.0f}\n")
            f.write(f"ratio to algorithmic: {stot / alg:.3f} (the rest is the fp32 partials, written and read "
                    f"once)\n")
            f.write(f"source_sha256: {_src_hash(*_SOURCES['split'])}\n")
        print("wrote", out)
    if len(mres) == 2:
        out = os.path.join(ROOT, "profiles", "mask_convert_16x4096x4096_counters.txt")
        total = 0.0
        with open(out, "w") as f:
            f.write(f"workload: bool mask {list(MASK_SHAPE)} -> bf16 additive\n")
            f.write("commands: as for prefill_gqa_causal_bf16_counters.txt (the counters pass ends with 6 mask "
                    "conversions)\n")
            for counter in ("FETCH_SIZE", "WRITE_SIZE"):
                kib_copy, factor, _, cname = res[counter]
                kib, n = mres[counter]
                b = kib * 1024.0 * factor
                total += b
                f.write(f"{counter}: scale factor {factor:.4f} ({cname}); mask_convert_kernel: {kib:.1f} "
                        f"KiB/dispatch over {n} dispatches -> {b:.0f} B\n")
            alg = 3 * int(np.prod(MASK_SHAPE))
            f.write(f"algorithmic bytes per call (mask read once, additive mask written once): {alg}\n")
            f.write(f"hbm_bytes_per_launch: {total:.0f}\n")
            f.write(f"ratio to algorithmic: {total / alg:.3f}\n")
            f.write(f"source_sha256: {_src_hash(*_SOURCES['mask'])}\n")
        print("wrote", out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters-pass", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-sq", metavar="DIR")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the attention path "
              "shards by heads with no communication; the sharding plan is written up with the design)",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        return _summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return _summarize_counters(*args.summarize_counters)
    if args.summarize_sq:
        return _summarize_sq(args.summarize_sq)
    if args.counters_pass:
        return _counters_pass()

    import numpy as np
    import torch

    import attention_flash_sdpa_amd as sdpa
    from attention_flash_sdpa_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sdpa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    ncu = props.multi_processor_count

    # ---------------- headline: causal GQA bf16 prefill ----------------
    w = inputs.WORKLOADS["gqa_causal_prefill_bf16"]
    q, k, v, _ = inputs.make_qkv(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty(w.batch, w.q_len, w.head_q, w.d_v, dtype=torch.bfloat16, device=dev)

    def step(i):
        sdpa.prefill(qd, kd, vd, scale=w.scale, causal=True, out=out)

    eager_ms = _time(step, args.steps, args.warmup, stream)
    ms = _graph_time(step, args.steps, args.warmup)
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    plan = sdpa.plan(_problem(sdpa, w), num_cus=ncu)

    # sampled parity of the timed output against the oracle
    import oracle

    rows = np.array([(0, i, h) for i in (0, 1, 255, 511) for h in (0, 13, 31)], dtype=np.int64)
    ref = oracle.sdpa(q, k, v, scale=w.scale, causal=True, rows=rows, want_lse=False)["out"]
    got = out.cpu()[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    prefill_err = float(np.abs(got - ref).max())
    prefill_nan = int(np.isnan(got).sum())

    _progress("prefill leg done")
    # ---------------- split-KV decode, 4 rotating K/V sets ----------------
    dw = inputs.WORKLOADS["splitkv_decode_bf16"]
    dq, dk0, dv0, _ = inputs.make_qkv(dw)
    dqd = dq.reshape(dw.batch, dw.head_q, dw.d_qk).to(dev)
    # every rotating K/V set is drawn by the seeded CPU recipe (seed + 100 * set)
    cpu_sets = [(dk0, dv0)] + [inputs.make_qkv(dw, kv_set=s_)[1:3] for s_ in range(1, dw.kv_sets)]
    sets = [(kk.to(dev), vv.to(dev)) for kk, vv in cpu_sets]
    dout = torch.empty(dw.batch, dw.head_q, dw.d_v, dtype=torch.bfloat16, device=dev)
    ws = sdpa.decode_workspace(dqd, sets[0][0], sets[0][1])

    def dstep(i):
        kk, vv = sets[i % len(sets)]
        sdpa.decode(dqd, kk, vv, scale=dw.scale, out=dout, workspace=ws)

    deager_ms = _time(dstep, args.decode_steps, args.warmup, stream)
    dms = _graph_time(dstep, args.decode_steps, args.warmup, period=len(sets))
    dbytes = dw.bytes_moved()
    dgbs = dbytes / (dms * 1e-3) / 1e9
    dplan = sdpa.plan(_problem(sdpa, dw), decode=True, num_cus=ncu)
    # streaming-read ceiling: the library's read probe over the same K and V
    # bytes, rotating over the same sets (two launches per set: K, then V)
    sink = torch.empty(2048, dtype=torch.int32, device=dev)

    def rstep(i):
        kk, vv = sets[i % len(sets)]
        sdpa.hbm_read_probe(kk, sink=sink)
        sdpa.hbm_read_probe(vv, sink=sink)

    rms = _graph_time(rstep, args.decode_steps, args.warmup, period=len(sets))
    rbytes = sum(t.numel() * t.element_size() for t in sets[0])
    read_gbs = rbytes / (rms * 1e-3) / 1e9
    # sampled parity of every set against the oracle
    drows = np.array([(b, 0, h) for b in (0, 7, 15) for h in (0, 17, 31)], dtype=np.int64)
    decode_err = 0.0
    decode_nan = 0
    for s_, (kk, vv) in enumerate(sets):
        sdpa.decode(dqd, kk, vv, scale=dw.scale, out=dout, workspace=ws)
        torch.cuda.synchronize()
        dref = oracle.sdpa(dq, cpu_sets[s_][0], cpu_sets[s_][1], scale=dw.scale, causal=False, rows=drows,
                           want_lse=False)["out"]
        dgot = dout.cpu()[drows[:, 0], drows[:, 2]].double().numpy()
        decode_err = max(decode_err, float(np.abs(dgot - dref).max()))
        decode_nan += int(np.isnan(dgot).sum())
    del sets
    dcpu = None
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        oracle.sdpa(dq, dk0, dv0, scale=dw.scale, causal=False, want_lse=False, threads=threads)
        sec = time.perf_counter() - t0
        dcpu = _cpu_line(round(dbytes / sec / 1e9, 3), "GB/s", threads,
                         f"whole decode workload ({dw.batch * dw.head_q} rows x {dw.kv_len} keys) in {sec:.2f} s, fp64")

    _progress("decode leg done")
    # ------- the same decode over a paged cache: 64- and 16-key pages, shuffled -------
    from oracle import paged as opaged

    paged_lines = {}
    for PS in (64, 16):
        P = dw.kv_len // PS
        kp0, vp0, table0 = inputs.paginate(dk0, dv0, PS, seed=dw.seed + 1)
        psets = [(kp0.to(dev), vp0.to(dev), table0.to(dev))]
        for s_ in range(1, dw.kv_sets):
            pk, pv, pt = inputs.paginate(cpu_sets[s_][0], cpu_sets[s_][1], PS, seed=dw.seed + 100 * s_ + 1)
            psets.append((pk.to(dev), pv.to(dev), pt.to(dev)))
            del pk, pv
        full = torch.full((dw.batch,), dw.kv_len, dtype=torch.int32, device=dev)

        def pstep(i):
            pk, pv, pt = psets[i % len(psets)]
            sdpa.decode_paged(dqd, pk, pv, page_table=pt, seq_lens=full, scale=dw.scale, out=dout, workspace=ws)

        peager_ms = _time(pstep, args.decode_steps, args.warmup, stream)
        pms = _graph_time(pstep, args.decode_steps, args.warmup, period=len(psets))
        pbytes = dbytes + table0.numel() * 4 + dw.batch * 4
        pgbs = pbytes / (pms * 1e-3) / 1e9
        # sets 1-3: sampled rows against the dense oracle of the same keys
        paged_err_rest = 0.0
        for s_ in range(1, len(psets)):
            pstep(s_)
            torch.cuda.synchronize()
            pref_s = oracle.sdpa(dq, cpu_sets[s_][0], cpu_sets[s_][1], scale=dw.scale, causal=False, rows=drows,
                                 want_lse=False)["out"]
            pgot = dout.cpu()[drows[:, 0], drows[:, 2]].double().numpy()
            paged_err_rest = max(paged_err_rest, float(np.abs(pgot - pref_s).max()))
        pstep(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pref = opaged.decode_paged(dq.reshape(dw.batch, dw.head_q, dw.d_qk), kp0, vp0, page_table=table0,
                                   page_size=PS, seq_lens=None, scale=dw.scale)["out"]
        psec = time.perf_counter() - t0
        paged_err = float(np.abs(dout.double().cpu().numpy() - pref).max())
        del psets, kp0, vp0
        paged_lines[PS] = {
            "workload": f"{dw.name} in {PS}-key pages (shuffled physical order, every sequence full)",
            "value": round(pgbs, 2), "unit": "GB/s", "ms_per_call": round(pms, 6),
            "eager_ms_per_call": round(peager_ms, 6), "steps": args.decode_steps, "kv_sets": dw.kv_sets,
            "algorithmic_bytes": pbytes,
            "roofline": {"bound": "hbm", "achieved": round(pgbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(pgbs / PEAK_HBM_GBS, 5),
                         "traffic": _traffic(f"decode_paged{PS}_splitkv_bf16_counters.txt", _SOURCES["decode"])},
            "parity": {"max_abs_err": max(paged_err, paged_err_rest),
                       "set0": {"max_abs_err": paged_err, "rows": dw.batch * dw.head_q},
                       "sets1_3": {"max_abs_err": paged_err_rest, "rows_per_set": int(len(drows))}},
            "cpu_baseline": _cpu_line(round(pbytes / psec / 1e9, 3), "GB/s", torch.get_num_threads(),
                                      f"whole workload through the paged oracle in {psec:.2f} s, fp64"),
        }

    del cpu_sets

    _progress("paged decode legs done")
    # ---------------- other prefill workloads (context lines) ----------------
    extra = {}
    for name in ("single_head_f16_128", "unaligned_full_bf16", "tiny_causal_bf16", "mla_fp8_causal_prefill"):
        xw = inputs.WORKLOADS[name]
        xq, xk, xv, xds = inputs.make_qkv(xw)
        xq, xk, xv = (t.to(dev) for t in (xq, xk, xv))
        odt = torch.bfloat16 if xw.out_dtype == "bf16" else torch.float16
        xo = torch.empty(xw.batch, xw.q_len, xw.head_q, xw.d_v, dtype=odt, device=dev)
        n = 100 if xw.flops() < 1e9 else max(args.steps // 4, MIN_LEG_CALLS)

        def xstep(i):
            sdpa.prefill(xq, xk, xv, scale=xw.scale, causal=xw.causal, out=xo, descale=xds)

        xeager = _time(xstep, n, args.warmup, stream)
        xms = _graph_time(xstep, n, args.warmup)
        xt = xw.flops() / (xms * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if xw.dtype == "fp8_e4m3" else PEAK_BF16_TFLOPS
        extra[name] = {"value": round(xt, 3), "unit": "TFLOP/s", "ms_per_call": round(xms, 6),
                       "eager_ms_per_call": round(xeager, 6), "steps": n,
                       "algorithmic_gflop": round(xw.flops() / 1e9, 4), "peak": peak,
                       "frac_of_peak": round(xt / peak, 5)}
        del xq, xk, xv, xo
    _progress("other prefill workloads done")
    # ------- cached-KV (chunked) prefill: 512 new queries/keys over 3584 cached -------
    from oracle import cached as ocached

    cw = CACHED_CHUNK
    g = torch.Generator().manual_seed(cw.seed)
    new = cw.kv_len - CACHED_LEN
    cq = torch.randn(1, cw.q_len, cw.head_q, cw.d_qk, generator=g).to(torch.bfloat16)
    ckc, cvc, ck, cv = (torch.randn(1, n, cw.head_kv, cw.d_qk, generator=g).to(torch.bfloat16)
                        for n in (CACHED_LEN, CACHED_LEN, new, new))
    cqd, ckcd, cvcd, ckd, cvd = (t.to(dev) for t in (cq, ckc, cvc, ck, cv))
    co = torch.empty(1, cw.q_len, cw.head_q, cw.d_v, dtype=torch.bfloat16, device=dev)

    def cstep(i):
        sdpa.prefill_cached(cqd, ckcd, cvcd, ckd, cvd, cache_len=CACHED_LEN, causal=True, scale=cw.scale, out=co)

    cn = max(args.steps // 4, MIN_LEG_CALLS)
    ceager = _time(cstep, cn, args.warmup, stream)
    cms = _graph_time(cstep, cn, args.warmup)
    cstep(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cref = ocached.prefill_cached(cq, ckc, cvc, ck, cv, cache_len=CACHED_LEN, scale=cw.scale, causal=True)["out"]
    csec = time.perf_counter() - t0
    cerr = float(np.abs(co.double().cpu().numpy() - cref).max())
    ct = cw.flops() / (cms * 1e-3) / 1e12
    cached_line = {"workload": f"{cw.q_len}-query chunk over {CACHED_LEN} cached keys, Hq {cw.head_q} / Hkv "
                               f"{cw.head_kv}, d {cw.d_qk}, bf16, causal on the new keys",
                   "value": round(ct, 3), "unit": "TFLOP/s", "ms_per_call": round(cms, 6),
                   "eager_ms_per_call": round(ceager, 6), "steps": cn,
                   "algorithmic_gflop": round(cw.flops() / 1e9, 4), "peak": PEAK_BF16_TFLOPS,
                   "frac_of_peak": round(ct / PEAK_BF16_TFLOPS, 5),
                   "parity": {"max_abs_err": cerr},
                   "cpu_baseline": _cpu_line(round(cw.flops() / csec / 1e12, 6), "TFLOP/s", torch.get_num_threads(),
                                             f"whole chunk through the cached-prefill oracle in {csec:.2f} s, "
                                             f"fp64")}
    del cqd, ckcd, cvcd, ckd, cvd

    _progress("cached prefill leg done")
    # ------- short chunk over long keys: the split across workgroups -------
    sw = SPLIT_CHUNK
    g = torch.Generator().manual_seed(sw.seed)
    sq = torch.randn(sw.batch, sw.q_len, sw.head_q, sw.d_qk, generator=g).to(torch.bfloat16)
    s_sets_cpu = [tuple(torch.randn(sw.batch, sw.kv_len, sw.head_kv, sw.d_qk, generator=g).to(torch.bfloat16)
                        for _ in range(2)) for _ in range(sw.kv_sets)]
    sqd = sq.to(dev)
    s_sets = [(a_.to(dev), b_.to(dev)) for a_, b_ in s_sets_cpu]
    so = torch.empty(sw.batch, sw.q_len, sw.head_q, sw.d_v, dtype=torch.bfloat16, device=dev)
    splan = sdpa.plan(_problem(sdpa, sw), num_cus=ncu)
    sws = torch.empty(max(splan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    s_none = torch.empty(0, dtype=torch.uint8, device=dev)

    def sstep(i, ws_=sws):
        kk, vv = s_sets[i % len(s_sets)]
        sdpa.prefill(sqd, kk, vv, causal=True, scale=sw.scale, out=so, workspace=ws_)

    sn = max(args.steps // 4, MIN_LEG_CALLS * sw.kv_sets)
    seager = _time(sstep, sn, args.warmup, stream)
    sms = _graph_time(sstep, sn, args.warmup, period=sw.kv_sets)
    s1ms = _graph_time(lambda i: sstep(i, s_none), sn, args.warmup, period=sw.kv_sets)
    sstep(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sref = oracle.sdpa(sq, *s_sets_cpu[0], scale=sw.scale, causal=True, want_lse=False)["out"]
    ssec = time.perf_counter() - t0
    serr = float(np.abs(so.double().cpu().numpy() - sref).max())
    snan = int(torch.isnan(so.float()).sum().item())
    sgbs = sw.bytes_moved() / (sms * 1e-3) / 1e9
    split_line = {"workload": f"{sw.q_len}-query chunk over {sw.kv_len} keys, Hq {sw.head_q} / Hkv {sw.head_kv}, "
                              f"d {sw.d_qk}, bf16, causal; {sw.kv_sets} rotating K/V sets "
                              f"({sw.kv_sets * 2 * sw.kv_len * sw.head_kv * sw.d_qk * 2 >> 20} MiB, past the "
                              f"256 MiB last-level cache)",
                  "value": round(sgbs, 2), "unit": "GB/s", "ms_per_call": round(sms, 6),
                  "eager_ms_per_call": round(seager, 6), "steps": _graph_chunk(sn, sw.kv_sets)[0],
                  "kv_splits": splan.kv_splits, "key_ranges_per_group": splan.num_splits,
                  "grid": splan.num_groups, "workspace_bytes": splan.workspace_bytes,
                  "unsplit_ms_per_call": round(s1ms, 6), "speedup_over_unsplit": round(s1ms / sms, 3),
                  "tflops": round(sw.flops() / (sms * 1e-3) / 1e12, 3),
                  "algorithmic_bytes": sw.bytes_moved(),
                  "roofline": {"bound": "hbm", "achieved": round(sgbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(sgbs / PEAK_HBM_GBS, 5),
                               "traffic": _traffic(SPLIT_COUNTERS, _SOURCES["split"])},
                  "parity": {"max_abs_err": serr, "nan": snan, "rows": sw.q_len * sw.head_q},
                  "cpu_baseline": _cpu_line(round(sw.bytes_moved() / ssec / 1e9, 3), "GB/s",
                                            torch.get_num_threads(),
                                            f"whole chunk (one K/V set) through the oracle in {ssec:.2f} s, fp64")}
    del sqd, s_sets, sws
    _progress("split prefill leg done")
    # ------- boolean -> additive mask conversion, 4 rotating buffer sets -------
    from oracle import mask as omask

    mshape = MASK_SHAPE
    mn = int(np.prod(mshape))
    msets = []
    for s_ in range(4):
        g = torch.Generator(device=dev).manual_seed(1007 + 100 * s_)
        msets.append(((torch.rand(mshape, generator=g, device=dev) < 0.5),
                      torch.empty(mshape, dtype=torch.bfloat16, device=dev)))

    def mstep(i):
        mm, mo = msets[i % len(msets)]
        sdpa.mask_convert(mm, out=mo)

    mms = _graph_time(mstep, args.decode_steps, args.warmup, period=len(msets))
    mbytes = 3 * mn
    mgbs = mbytes / (mms * 1e-3) / 1e9
    mstep(0)
    torch.cuda.synchronize()
    msample = msets[0][0][0].cpu().numpy().astype(np.uint8)
    t0 = time.perf_counter()
    omask.mask_convert(msample, "bf16")
    msec = time.perf_counter() - t0
    mrows = slice(0, 64)
    mref = omask.mask_convert(msets[0][0][0, mrows].cpu().numpy().astype(np.uint8), "bf16")
    mexact = bool(np.array_equal(msets[0][1][0, mrows].view(torch.int16).cpu().numpy().view(np.uint16), mref))
    # the same HBM traffic as a plain device-to-device copy (read and write
    # 1.5 bytes per mask element each), rotating four buffer pairs: what the
    # memory system gives a kernel that does nothing else
    csets = [(torch.empty(mbytes // 2, dtype=torch.uint8, device=dev).fill_(s_),
              torch.empty(mbytes // 2, dtype=torch.uint8, device=dev)) for s_ in range(4)]

    def cstep(i):
        src, dst = csets[i % len(csets)]
        dst.copy_(src)

    cms = _time(cstep, max(MIN_LEG_CALLS, args.decode_steps // 4), max(4, args.warmup), torch.cuda.current_stream())
    copy_ceiling = {"value": round(mbytes / (cms * 1e-3) / 1e9, 2), "unit": "GB/s", "ms_per_copy": round(cms, 6),
                    "bytes": mbytes, "frac_of_it": round(mgbs / (mbytes / (cms * 1e-3) / 1e9), 5),
                    "method": "torch copy_ of half the conversion's bytes (its read plus write are the "
                              "conversion's traffic), four rotating buffer pairs, back-to-back eager calls"}
    del csets
    mask_line = {"workload": f"bool mask {list(mshape)} -> bf16 additive", "value": round(mgbs, 2), "unit": "GB/s",
                 "ms_per_call": round(mms, 6), "steps": args.decode_steps, "buffer_sets": len(msets),
                 "algorithmic_bytes": mbytes,
                 "roofline": {"bound": "hbm", "achieved": round(mgbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(mgbs / PEAK_HBM_GBS, 5),
                              "traffic": _traffic("mask_convert_16x4096x4096_counters.txt", _SOURCES["mask"])},
                 "copy_ceiling": copy_ceiling,
                 "parity": {"bit_exact_rows": 64, "exact": mexact},
                 "cpu_baseline": _cpu_line(round(3 * msample.size / msec / 1e9, 3), "GB/s", 1,
                                           f"one [{MASK_SHAPE[1]}, {MASK_SHAPE[2]}] slice ({msample.size} elements) "
                                           f"through the numpy oracle in {msec:.2f} s")}
    del msets

    _progress("mask conversion leg done")
    # ------- prefill with a full additive mask (per-head bias) -------
    from oracle import mask as omask2

    xw = MASKED
    mqd, mkd, mvd, mbias = _masked_inputs(dev)
    mq, mk, mv = (t.cpu() for t in (mqd, mkd, mvd))
    mo = torch.empty(1, xw.q_len, xw.head_q, xw.d_v, dtype=torch.bfloat16, device=dev)

    def xmstep(i):
        sdpa.prefill_masked(mqd, mkd, mvd, mbias, scale=xw.scale, out=mo)

    xn = max(args.steps // 10, MIN_LEG_CALLS)
    xmms = _graph_time(xmstep, xn, args.warmup)
    xmstep(0)
    torch.cuda.synchronize()
    G = xw.head_q // xw.head_kv
    mb_cpu = mbias[:, :G].cpu()
    t0 = time.perf_counter()
    mref = omask2.prefill_masked(mq[:, :, :G], mk[:, :, :1], mv[:, :, :1], mb_cpu, scale=xw.scale,
                                 causal=False)["out"]
    xsec = time.perf_counter() - t0
    merr = float(np.abs(mo[:, :, :G].double().cpu().numpy() - mref).max())
    xt = xw.flops() / (xmms * 1e-3) / 1e12
    masked_line = {"workload": f"{xw.q_len} x {xw.kv_len}, Hq {xw.head_q} / Hkv {xw.head_kv}, d {xw.d_qk}, bf16, "
                               f"per-head additive bias [1, {xw.head_q}, {xw.q_len}, {xw.kv_len}]",
                   "value": round(xt, 3), "unit": "TFLOP/s", "ms_per_call": round(xmms, 6), "steps": xn,
                   "algorithmic_gflop": round(xw.flops() / 1e9, 4), "peak": PEAK_BF16_TFLOPS,
                   "frac_of_peak": round(xt / PEAK_BF16_TFLOPS, 5),
                   "mask_bytes": int(mbias.numel() * 2), "parity": {"max_abs_err": merr, "heads_checked": G},
                   "cpu_baseline": _cpu_line(round(xw.flops() * G / xw.head_q / xsec / 1e12, 6), "TFLOP/s",
                                             torch.get_num_threads(),
                                             f"{G} of {xw.head_q} heads (one GQA group) through the masked "
                                             f"oracle in {xsec:.2f} s, fp64")}
    del mqd, mkd, mvd, mbias, mo

    # launch floor: a one-element device op, eager and replayed from a graph
    one = torch.zeros(1, device=dev)
    floor_eager = _time(lambda i: one.add_(1.0), args.steps, args.warmup, stream)
    floor_graph = _graph_time(lambda i: one.add_(1.0), args.steps, args.warmup)

    _progress("masked prefill leg done")
    # ---------------- CPU baseline: the oracle on the host cores ----------------
    cpu = None
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        oracle.sdpa(q, k, v, scale=w.scale, causal=True, want_lse=False, threads=threads)
        sec = time.perf_counter() - t0
        cpu = {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"whole causal GQA prefill workload ({w.batch * w.q_len * w.head_q} query rows, "
                         f"{flops / 1e9:.2f} GFLOP) in {sec:.2f} s, fp64, {_cpu_model()}"}

    traffic = _traffic("prefill_gqa_causal_bf16_counters.txt", _SOURCES["prefill"])
    dtraffic = _traffic("decode_splitkv_bf16_counters.txt", _SOURCES["decode"])
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
                   "algorithmic_gflop": round(flops / 1e9, 4), "grid": plan.num_groups,
                   "key_ranges_per_group": plan.num_splits,
                   "range_iters": {"max": plan.range_iters_max, "min": plan.range_iters_min,
                                   "mean": round(plan.range_iters_sum / (plan.num_groups * plan.num_splits), 3),
                                   "imbalance": round(plan.imbalance(), 3)},
                   "launch": "hip graph replays of a captured chunk of calls (chunk divides steps; at least one "
                             "untimed replay first)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 5), "traffic": traffic},
        "cpu_baseline": cpu,
        "eager": {"ms_per_step": round(eager_ms, 6), "value": round(flops / (eager_ms * 1e-3) / 1e12, 3)},
        "parity": {"max_abs_err": prefill_err, "nan": prefill_nan, "sampled_rows": int(len(rows))},
        "decode": {
            "workload": dw.name, "value": round(dgbs, 2), "unit": "GB/s", "ms_per_call": round(dms, 6),
            "eager_ms_per_call": round(deager_ms, 6),
            "steps": args.decode_steps, "kv_sets": dw.kv_sets, "num_splits": dplan.num_splits,
            "algorithmic_bytes": dbytes,
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dgbs / PEAK_HBM_GBS, 5), "traffic": dtraffic},
            "read_ceiling": {"value": round(read_gbs, 2), "unit": "GB/s", "ms_per_set": round(rms, 6),
                             "bytes": rbytes, "frac_of_it": round(dgbs / read_gbs, 5),
                             "method": "sdpa_hbm_read_probe (16-byte non-temporal loads) over the same K and V, "
                                       "rotating sets, two launches per set, graph replays"},
            "parity": {"max_abs_err": decode_err, "nan": decode_nan, "sets_checked": dw.kv_sets,
                       "rows_per_set": int(len(drows))},
            "cpu_baseline": dcpu,
        },
        "decode_paged": paged_lines[64],
        "decode_paged_16": paged_lines[16],
        "prefill_cached": cached_line,
        "prefill_split": split_line,
        "mask_convert": mask_line,
        "prefill_masked": masked_line,
        "other_workloads": extra,
        "launch_floor_us": {"eager": round(floor_eager * 1e3, 3), "graph": round(floor_graph * 1e3, 3)},
        "device": {"name": props.name, "cus": ncu},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
