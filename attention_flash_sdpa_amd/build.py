"""Builds the HIP shared library libsdpa_mi355x.so in-tree for gfx950.

    python -m attention_flash_sdpa_amd.build [--isa]

Every source is compiled with hipcc; HIP device code is built for gfx950 only
and with packed-fp32 instruction selection disabled.  ``--isa`` also keeps the
device assembly (``_build/*.s``) and prints the per-kernel resource usage
(VGPR/AGPR counts, scratch, occupancy) reported by the compiler.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsdpa_mi355x.so")
SOURCES = ["sdpa_abi.cpp", "planner.cpp", "prefill.hip", "prefill_cached.hip", "prefill_split.hip",
           "prefill_o2.hip", "prefill_fp8.hip", "decode.hip", "mask.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fgpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]


# Per-source backend options.  The one-wave-per-SIMD prefill kernels use both
# register files: MFMA results stay in VGPRs (the softmax reads the scores with
# VALU instructions), AGPRs take what does not fit.
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "prefill_cached.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "prefill_split.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, isa: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        if isa:
            cmd += ["-Rpass-analysis=kernel-resource-usage", "-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return out


def build(isa: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        outs = list(ex.map(lambda s: _compile(s, isa), SOURCES))
    if verbose or isa:
        for s, o in zip(SOURCES, outs):
            if o.strip():
                print(f"--- {s}\n{o}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[os.path.join(BUILD, s + ".o") for s in SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(isa="--isa" in sys.argv, verbose=True))
