"""fp64 CPU oracle for scaled-dot-product attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Two parts:

* ``sdpa()`` -- ctypes front end of ``sdpa_oracle.c``, the plain two-pass fp64
  definition softmax(Q K^T * scale + mask) V evaluated row by row (page
  "Xe SDPA Forward Mainloop -- Key Loops + Shapes", section "Full simplified
  pseudocode", which streams the same result block by block).
* ``blocked.py`` -- the blocked online-softmax algorithm of that same section,
  with the split-KV combine of the two-phase decode ("xe2-sdp-kernels",
  section "Assets"), in fp64 numpy; used only to show that the method's
  rescale algebra reproduces the definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdpa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_sdpa_oracle.so")

# dtype codes understood by the C oracle
F16, BF16, FP8_E4M3, F32, F64 = 0, 1, 2, 3, 4

_lib = None


def build(force: bool = True) -> str:
    """Compiles the C oracle with gcc (OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_sdpa_rows.restype = ctypes.c_int
    lib.orc_sdpa_rows.argtypes = (
        [ctypes.c_int] * 9
        + [ctypes.c_void_p] * 3
        + [ctypes.c_double] * 4
        + [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    )
    for name in ("orc_decode_f16", "orc_decode_bf16"):
        getattr(lib, name).restype = ctypes.c_double
        getattr(lib, name).argtypes = [ctypes.c_uint16]
    lib.orc_decode_e4m3.restype = ctypes.c_double
    lib.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return _load().orc_max_threads()


def _as_bits(x):
    """(contiguous numpy array of raw element bits, oracle dtype code)."""
    import torch

    if isinstance(x, np.ndarray):
        if x.dtype == np.float64:
            return np.ascontiguousarray(x), F64
        if x.dtype == np.float32:
            return np.ascontiguousarray(x), F32
        raise TypeError(f"unsupported numpy dtype {x.dtype}")
    t = x.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), BF16
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16), F16
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy(), FP8_E4M3
    if t.dtype == torch.float32:
        return t.numpy(), F32
    if t.dtype == torch.float64:
        return t.numpy(), F64
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def sdpa(q, k, v, *, scale: float, causal: bool, descale=(1.0, 1.0, 1.0), rows=None,
         want_lse: bool = True, want_probs: bool = False, threads: int = 0):
    """fp64 attention on the dequantised inputs.

    q: [B, Sq, Hq, D]; k: [B, Sk, Hkv, D]; v: [B, Sk, Hkv, Dv] as torch tensors
    (bf16 / fp16 / fp8 e4m3fn / fp32 / fp64) or float32/float64 numpy arrays.
    ``descale`` holds the per-tensor dequantisation factors (q, k, v).
    ``rows``: optional int array [n, 3] of (b, i, h) triples to evaluate.

    Returns a dict with ``out`` ([B, Sq, Hq, Dv], or [n, Dv] when rows are given),
    ``lse`` ([B, Hq, Sq] natural log, or [n]) and optionally ``probs``
    ([B, Sq, Hq, Sk] or [n, Sk]).
    """
    lib = _load()
    B, Sq, Hq, D = (int(s) for s in q.shape)
    Bk, Sk, Hkv, Dk = (int(s) for s in k.shape)
    Dv = int(v.shape[-1])
    if Bk != B or Dk != D or tuple(int(s) for s in v.shape[:3]) != (B, Sk, Hkv) or Hq % Hkv:
        raise ValueError("inconsistent q/k/v shapes")
    qb, qdt = _as_bits(q)
    kb, kdt = _as_bits(k)
    vb, vdt = _as_bits(v)
    if kdt != vdt:
        raise TypeError("k and v must share a dtype")
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        rows_ptr = rows.ctypes.data
    else:
        n = B * Sq * Hq
        rows_ptr = None
    out = np.zeros((n, Dv), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64) if want_lse else None
    probs = np.zeros((n, Sk), dtype=np.float64) if want_probs else None
    rc = lib.orc_sdpa_rows(
        B, Sq, Sk, Hq, Hkv, D, Dv, qdt, kdt,
        qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
        float(descale[0]), float(descale[1]), float(descale[2]), float(scale), int(bool(causal)),
        n, rows_ptr, out.ctypes.data,
        lse.ctypes.data if lse is not None else None,
        probs.ctypes.data if probs is not None else None,
        int(threads),
    )
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    res = {}
    if rows is None:
        res["out"] = out.reshape(B, Sq, Hq, Dv)
        if lse is not None:
            res["lse"] = lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()
        if probs is not None:
            res["probs"] = probs.reshape(B, Sq, Hq, Sk)
    else:
        res["out"] = out
        if lse is not None:
            res["lse"] = lse
        if probs is not None:
            res["probs"] = probs
    return res


def decode_scalar(code: int, bits: int) -> float:
    """Widens one raw element (oracle dtype code) to a Python float."""
    lib = _load()
    if code == F16:
        return lib.orc_decode_f16(bits)
    if code == BF16:
        return lib.orc_decode_bf16(bits)
    if code == FP8_E4M3:
        return lib.orc_decode_e4m3(bits)
    raise ValueError(code)
