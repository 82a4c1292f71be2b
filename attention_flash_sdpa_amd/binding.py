"""ctypes binding of libsdpa_mi355x.so (the C ABI in include/sdpa.h).

Argument marshalling only: every step of attention runs in the HIP kernels.
PyTorch supplies device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing, importing the entry points raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdpa_mi355x.so")

F16, BF16, FP8_E4M3 = 0, 1, 2
STATUS = {
    0: "SDPA_OK", 1: "SDPA_ERR_NULL_PTR", 2: "SDPA_ERR_BAD_SHAPE", 3: "SDPA_ERR_BAD_SCALE",
    4: "SDPA_ERR_UNSUPPORTED", 5: "SDPA_ERR_MISALIGNED", 6: "SDPA_ERR_WORKSPACE", 7: "SDPA_ERR_HIP",
}

# every symbol include/sdpa.h declares
EXPORTS = (
    "sdpa_abi_version", "sdpa_status_string", "sdpa_last_error", "sdpa_plan",
    "sdpa_prefill_workspace_bytes", "sdpa_decode_workspace_bytes", "sdpa_prefill_fwd", "sdpa_decode_fwd",
    "sdpa_decode_paged_fwd", "sdpa_prefill_cached_fwd", "sdpa_mask_convert", "sdpa_prefill_masked_fwd",
    "sdpa_loop_counts", "sdpa_set_prefill_variant", "sdpa_decode_fwd_noalloc", "sdpa_hbm_read_probe",
    "sdpa_prefill_cached_workspace_bytes",
)


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("head_q", ctypes.c_int32), ("head_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float), ("q_descale", ctypes.c_float),
        ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
    ]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "waves_per_group", "rows_per_wave", "heads_per_group", "qtiles_per_group", "block_q",
        "block_k", "stages", "q_tiles", "kv_blocks", "num_groups", "num_splits", "blocks_per_split",
        "combine_groups")] + [("lds_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                              ("range_iters_sum", ctypes.c_int64), ("range_iters_max", ctypes.c_int32),
                              ("range_iters_min", ctypes.c_int32), ("kv_splits", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def imbalance(self) -> float:
        """Busiest key range's iterations over the mean of all ranges (1 = even;
        prefill plans only)."""
        ranges = self.num_groups * self.num_splits  # num_groups counts the kv_splits workgroups
        return self.range_iters_max * ranges / self.range_iters_sum if self.range_iters_sum else 1.0


class LoopCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_blocks", "k_blocks", "d_loops", "vv_loops", "blocks_visited", "blocks_masked", "qk_tiles", "pv_tiles",
        "softmax_tiles")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class SdpaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Loads the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m attention_flash_sdpa_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.sdpa_abi_version.restype = ctypes.c_int
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_plan.restype = ctypes.c_int
    lib.sdpa_plan.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(Plan)]
    lib.sdpa_loop_counts.restype = ctypes.c_int
    lib.sdpa_loop_counts.argtypes = [ctypes.c_int] * 9 + [ctypes.POINTER(LoopCounts)]
    lib.sdpa_set_prefill_variant.restype = ctypes.c_int
    lib.sdpa_set_prefill_variant.argtypes = [ctypes.c_char_p]
    lib.sdpa_prefill_workspace_bytes.restype = sz
    lib.sdpa_prefill_workspace_bytes.argtypes = [P]
    lib.sdpa_prefill_cached_workspace_bytes.restype = sz
    lib.sdpa_prefill_cached_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.sdpa_decode_workspace_bytes.restype = sz
    lib.sdpa_decode_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.sdpa_prefill_fwd.restype = ctypes.c_int
    lib.sdpa_prefill_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_prefill_cached_fwd.restype = ctypes.c_int
    lib.sdpa_mask_convert.restype = ctypes.c_int
    lib.sdpa_prefill_masked_fwd.restype = ctypes.c_int
    lib.sdpa_prefill_masked_fwd.argtypes = [P, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, vp, vp,
                                            vp]
    lib.sdpa_mask_convert.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, vp]
    lib.sdpa_hbm_read_probe.restype = ctypes.c_int
    lib.sdpa_hbm_read_probe.argtypes = [vp, ctypes.c_int64, vp, vp]
    lib.sdpa_prefill_cached_fwd.argtypes = [P, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp, sz,
                                            vp]
    lib.sdpa_decode_fwd.restype = ctypes.c_int
    lib.sdpa_decode_fwd.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.sdpa_decode_fwd_noalloc.restype = ctypes.c_int
    lib.sdpa_decode_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    i32 = ctypes.c_int32
    lib.sdpa_decode_paged_fwd.restype = ctypes.c_int
    lib.sdpa_decode_paged_fwd.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise SdpaError(status, (load().sdpa_last_error() or b"").decode())


def _code_of(dtype) -> int:
    import torch

    m = {torch.float16: F16, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}
    if dtype not in m:
        raise TypeError(f"unsupported dtype {dtype}")
    return m[dtype]


def _dtype_code(t) -> int:
    return _code_of(t.dtype)


def make_problem(*, batch, q_len, kv_len, head_q, head_kv, d_qk, d_v, in_dtype, out_dtype, causal, scale,
                 descale=(1.0, 1.0, 1.0)) -> Problem:
    return Problem(int(batch), int(q_len), int(kv_len), int(head_q), int(head_kv), int(d_qk), int(d_v),
                   int(in_dtype), int(out_dtype), int(bool(causal)), float(scale), float(descale[0]),
                   float(descale[1]), float(descale[2]))


def plan(problem: Problem, *, decode: bool = False, num_cus: int = 0, num_splits: int = 0) -> Plan:
    out = Plan()
    _check(load().sdpa_plan(ctypes.byref(problem), int(decode), int(num_cus), int(num_splits), ctypes.byref(out)))
    return out


def loop_counts(*, q_len, kv_len, d_qk, d_v, block_q, block_k, block_d, block_v, causal) -> LoopCounts:
    out = LoopCounts()
    _check(load().sdpa_loop_counts(int(q_len), int(kv_len), int(d_qk), int(d_v), int(block_q), int(block_k),
                                   int(block_d), int(block_v), int(bool(causal)), ctypes.byref(out)))
    return out


def set_prefill_variant(name: str | None) -> None:
    """Forces one form of the 16-bit prefill kernels ("narrow1", "narrow2",
    "occ2", "split4", "kvsplit") for later calls in this process; None or ""
    restores the planner's choice.  For tuning sweeps and tests."""
    _check(load().sdpa_set_prefill_variant((name or "").encode()))


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_inputs(names, tensors, *, same_dtype=True):
    """Every input is a contiguous tensor on one device, with one dtype."""
    dev = tensors[0].device
    for n, t in zip(names, tensors):
        _require(t.is_cuda and t.is_contiguous(), f"{n} must be a contiguous device tensor")
        _require(t.device == dev, f"{n} is on {t.device}, {names[0]} on {dev}")
        if same_dtype:
            _require(t.dtype == tensors[0].dtype, f"{n} has dtype {t.dtype}, {names[0]} {tensors[0].dtype}")


def _check_output(name, t, shape, dtypes, device):
    """A caller's output buffer: exact shape, an accepted dtype, contiguous, on
    the inputs' device (the kernels write every element of that shape)."""
    if t is None:
        return
    _require(tuple(t.shape) == tuple(shape), f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.dtype in dtypes, f"{name} must have dtype in {[str(d) for d in dtypes]}, got {t.dtype}")
    _require(t.is_cuda and t.is_contiguous() and t.device == device,
             f"{name} must be a contiguous tensor on {device}")


def _check_prefill_shapes(q, k, v):
    """q [B, Sq, Hq, D], k [B, Sk, Hkv, D], v [B, Sk, Hkv, Dv]."""
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    _require(k.shape[0] == q.shape[0] and v.shape[0] == q.shape[0], "q, k, v must have the same batch")
    _require(k.shape[-1] == q.shape[-1], f"k head dim {k.shape[-1]} != q head dim {q.shape[-1]}")
    _require(v.shape[:3] == k.shape[:3], f"v {tuple(v.shape)} does not match k {tuple(k.shape)} in [B, Sk, Hkv]")


def _out_dtypes(q):
    import torch

    return (torch.bfloat16, torch.float16) if q.dtype == torch.float8_e4m3fn else (q.dtype,)


def prefill_workspace_bytes(q, k, v, *, causal=False, descale=(1.0, 1.0, 1.0), out_dtype=None) -> int:
    """Workspace bytes ``prefill`` uses for these shapes (0 unless the planner
    splits the key range across workgroups)."""
    import torch

    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if out_dtype is None:
        out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    pr = make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=v.shape[-1],
                      in_dtype=_dtype_code(q), out_dtype=_code_of(out_dtype), causal=causal, scale=1.0,
                      descale=descale)
    return int(load().sdpa_prefill_workspace_bytes(ctypes.byref(pr)))


def prefill(q, k, v, *, scale=None, causal=False, out=None, lse=None, descale=(1.0, 1.0, 1.0), out_dtype=None,
            workspace=None, stream=None):
    """O = softmax(Q K^T * scale + mask) V on the GPU.

    q [B, Sq, Hq, D], k [B, Sk, Hkv, D], v [B, Sk, Hkv, Dv] contiguous device
    tensors; returns O [B, Sq, Hq, Dv] (``out`` if given).  ``lse`` is an
    optional fp32 [B, Hq, Sq] tensor to receive the log-sum-exp.
    ``workspace``: a device uint8 tensor for the partials of a key range
    split across workgroups (``prefill_workspace_bytes``); None allocates one
    when the plan splits; a smaller one (an empty tensor included) runs the
    problem without that split."""
    import torch

    _check_inputs(("q", "k", "v"), (q, k, v))
    _check_prefill_shapes(q, k, v)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    Dv = v.shape[-1]
    if out_dtype is None:
        out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    _check_output("out", out, (B, Sq, Hq, Dv), _out_dtypes(q), q.device)
    _check_output("lse", lse, (B, Hq, Sq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Sq, Hq, Dv, dtype=out_dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=Dv,
                      in_dtype=_dtype_code(q), out_dtype=_dtype_code(out), causal=causal, scale=scale,
                      descale=descale)
    lib = load()
    ws, ws_bytes = _prefill_workspace(workspace, lib.sdpa_prefill_workspace_bytes(ctypes.byref(pr)), q.device)
    _check(lib.sdpa_prefill_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                                ws_bytes, _stream_handle(stream)))
    return out


def _prefill_workspace(workspace, need, device):
    """(tensor or None, bytes) for a prefill call: `workspace` as given (an
    empty one passes NULL), or a new one of `need` bytes when None."""
    import torch

    if workspace is None:
        return (torch.empty(need, dtype=torch.uint8, device=device) if need else None), need
    _require(workspace.dtype == torch.uint8 and workspace.is_contiguous() and workspace.device == device,
             "workspace must be a contiguous uint8 tensor on q's device")
    return (workspace if workspace.numel() else None), workspace.numel()


def prefill_cached_workspace_bytes(q, k, v, *, cache_len, causal=False) -> int:
    """Workspace bytes ``prefill_cached`` uses for a chunk (q, k, v: its
    queries and new keys) over ``cache_len`` cached keys (0 unless the
    planner splits the keys across workgroups)."""
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    pr = make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=v.shape[-1],
                      in_dtype=_dtype_code(q), out_dtype=_dtype_code(q), causal=causal, scale=1.0)
    return int(load().sdpa_prefill_cached_workspace_bytes(ctypes.byref(pr), int(cache_len)))


def prefill_cached(q, k_cache, v_cache, k, v, *, cache_len, scale=None, causal=False, out=None, lse=None,
                   workspace=None, stream=None):
    """Cached-KV (chunked) prefill (``sdpa_prefill_cached_fwd``): the chunk's
    queries q [B, Sq, Hq, D] attend to cache keys 0 .. cache_len-1 of
    k_cache / v_cache [B, cap, Hkv, D|Dv] followed by the chunk's own keys
    k / v [B, Sk, Hkv, D|Dv]; with ``causal`` only the new keys are masked
    (bottom-right, Sq <= Sk).  Returns O [B, Sq, Hq, Dv].  ``workspace`` as
    for ``prefill`` (``prefill_cached_workspace_bytes``)."""
    import torch

    _check_inputs(("q", "k_cache", "v_cache", "k", "v"), (q, k_cache, v_cache, k, v))
    _check_prefill_shapes(q, k, v)
    _require(k_cache.dim() == 4 and v_cache.dim() == 4, "k_cache, v_cache must be 4-D")
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    Dv = v.shape[-1]
    if k_cache.shape[0] != B or k_cache.shape[2:] != k.shape[2:] or v_cache.shape[:3] != k_cache.shape[:3] \
            or v_cache.shape[-1] != Dv or v.shape[:3] != k.shape[:3] or k.shape[0] != B or k.shape[-1] != D:
        raise ValueError(f"shapes disagree: q {tuple(q.shape)}, k_cache {tuple(k_cache.shape)}, "
                         f"v_cache {tuple(v_cache.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not 0 <= cache_len <= k_cache.shape[1]:
        raise ValueError(f"cache_len {cache_len} outside [0, {k_cache.shape[1]}]")
    _check_output("out", out, (B, Sq, Hq, Dv), (q.dtype,), q.device)
    _check_output("lse", lse, (B, Hq, Sq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Sq, Hq, Dv, dtype=q.dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=Dv,
                      in_dtype=_dtype_code(q), out_dtype=_dtype_code(out), causal=causal, scale=scale)
    lib = load()
    ws, ws_bytes = _prefill_workspace(workspace, lib.sdpa_prefill_cached_workspace_bytes(ctypes.byref(pr),
                                                                                         int(cache_len)), q.device)
    _check(lib.sdpa_prefill_cached_fwd(ctypes.byref(pr), _ptr(q), _ptr(k_cache), _ptr(v_cache), int(cache_len),
                                       int(k_cache.shape[1]), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                                       ws_bytes, _stream_handle(stream)))
    return out


@dataclass
class DecodeWorkspace:
    tensor: object
    nbytes: int


def decode_workspace(q, k, v, *, num_splits=0, descale=(1.0, 1.0, 1.0), kv_len=None):
    """Allocates the decode workspace for these shapes (reusable across calls);
    ``kv_len`` overrides the key count read from ``k`` (paged caches)."""
    import torch

    pr = _decode_problem(q, k, v, 1.0, descale, None, kv_len)
    plan(pr, decode=True, num_splits=num_splits)  # raises for an invalid problem
    n = load().sdpa_decode_workspace_bytes(ctypes.byref(pr), int(num_splits))
    # an empty batch needs none; keep a valid aligned pointer all the same
    return DecodeWorkspace(torch.empty(max(n, 256), dtype=torch.uint8, device=q.device), n)


def _decode_problem(q, k, v, scale, descale, out, kv_len=None):
    B, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if kv_len is not None:
        Sk = kv_len
    Dv = v.shape[-1]
    od = _dtype_code(out) if out is not None else _dtype_code(q)
    return make_problem(batch=B, q_len=1, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=Dv,
                        in_dtype=_dtype_code(q), out_dtype=od, causal=False, scale=scale, descale=descale)


def _check_caches(q, k, v, *, dense):
    """The kernels index K and V with one row geometry and read d_qk from q."""
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches 4-D")
    if k.shape[:3] != v.shape[:3] or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"cache shapes disagree: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if dense and k.shape[0] != q.shape[0]:
        raise ValueError("dense caches need one row of keys per sequence")


def decode(q, k, v, *, scale=None, out=None, lse=None, num_splits=0, workspace=None, descale=(1.0, 1.0, 1.0),
           stream=None):
    """Two-phase split-KV decode: q [B, Hq, D], k/v cache [B, Sk, Hkv, D|Dv];
    returns O [B, Hq, Dv].  ``lse`` is an optional fp32 [B, Hq] tensor."""
    import torch

    _check_inputs(("q", "k", "v"), (q, k, v))
    _check_caches(q, k, v, dense=True)
    B, Hq, D = q.shape
    Dv = v.shape[-1]
    _check_output("out", out, (B, Hq, Dv), (q.dtype,), q.device)
    _check_output("lse", lse, (B, Hq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Hq, Dv, dtype=q.dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = _decode_problem(q, k, v, scale, descale, out)
    lib = load()
    if workspace is None:
        workspace = decode_workspace(q, k, v, num_splits=num_splits, descale=descale)
    _require(workspace.tensor.device == q.device, "workspace must be on q's device")
    _check(lib.sdpa_decode_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(num_splits),
                               _ptr(workspace.tensor), workspace.nbytes, _stream_handle(stream)))
    return out


def decode_noalloc(q, k, v, *, scale=None, out=None, lse=None, num_splits=0, descale=(1.0, 1.0, 1.0), stream=None):
    """Two-phase split-KV decode through ``sdpa_decode_fwd_noalloc``: the
    split partials live in the library's static per-GPU scratch, so no
    workspace is allocated (``out`` is still allocated here when not given).
    Arguments as for ``decode``; calls that overlap on one GPU race."""
    import torch

    _check_inputs(("q", "k", "v"), (q, k, v))
    _check_caches(q, k, v, dense=True)
    B, Hq, D = q.shape
    Dv = v.shape[-1]
    _check_output("out", out, (B, Hq, Dv), (q.dtype,), q.device)
    _check_output("lse", lse, (B, Hq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Hq, Dv, dtype=q.dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = _decode_problem(q, k, v, scale, descale, out)
    _check(load().sdpa_decode_fwd_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                          int(num_splits), _stream_handle(stream)))
    return out


def decode_paged(q, k_cache, v_cache, *, page_table=None, seq_lens=None, kv_len=None, scale=None, out=None,
                 lse=None, num_splits=0, workspace=None, descale=(1.0, 1.0, 1.0), stream=None):
    """Decode over variable-length and/or paged caches (``sdpa_decode_paged_fwd``).

    q [B, Hq, D].  With ``page_table`` (int32 [B, pages_per_seq] on the
    device) the caches are pools [num_pages, page_size, Hkv, D|Dv] and
    ``kv_len`` (default pages_per_seq * page_size) bounds every sequence;
    without it they are dense [B, kv_len, Hkv, D|Dv].  ``seq_lens`` (int32
    [B] on the device, or None) gives each sequence's key count."""
    import torch

    _check_inputs(("q", "k_cache", "v_cache"), (q, k_cache, v_cache))
    B, Hq, D = q.shape
    Dv = v_cache.shape[-1]
    for t in (page_table, seq_lens):
        if t is not None and (not t.is_contiguous() or not t.is_cuda or t.device != q.device):
            raise ValueError("page_table and seq_lens must be contiguous tensors on q's device")
    for t in (page_table, seq_lens):
        if t is not None and t.dtype != torch.int32:
            raise TypeError("page_table and seq_lens must be int32")
    _check_caches(q, k_cache, v_cache, dense=page_table is None)
    if page_table is not None:
        num_pages, page_size = int(k_cache.shape[0]), int(k_cache.shape[1])
        pages_per_seq = int(page_table.shape[1])
        if page_table.shape[0] != B:
            raise ValueError("page_table must have one row per sequence")
        if kv_len is None:
            kv_len = pages_per_seq * page_size
    else:
        num_pages = page_size = pages_per_seq = 0
        kv_len = int(k_cache.shape[1]) if kv_len is None else kv_len
        if kv_len > k_cache.shape[1]:  # the dense cache is also the row stride: it must hold kv_len keys
            raise ValueError(f"kv_len {kv_len} exceeds the dense cache's {k_cache.shape[1]} keys")
    if seq_lens is not None and seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [B]")
    _check_output("out", out, (B, Hq, Dv), (q.dtype,), q.device)
    _check_output("lse", lse, (B, Hq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Hq, Dv, dtype=q.dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = _decode_problem(q, k_cache, v_cache, scale, descale, out, kv_len)
    lib = load()
    if workspace is None:
        workspace = decode_workspace(q, k_cache, v_cache, num_splits=num_splits, descale=descale, kv_len=kv_len)
    _require(workspace.tensor.device == q.device, "workspace must be on q's device")
    _check(lib.sdpa_decode_paged_fwd(ctypes.byref(pr), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                     _ptr(page_table), num_pages, page_size, pages_per_seq, _ptr(out), _ptr(lse),
                                     int(num_splits), _ptr(workspace.tensor), workspace.nbytes,
                                     _stream_handle(stream)))
    return out


def mask_convert(mask, *, out_dtype=None, out=None, stream=None):
    """Additive mask of a boolean (or uint8) device mask: 0 where the key
    takes part (nonzero), -inf where it does not; same shape, dtype
    ``out_dtype`` (torch.float16 or torch.bfloat16, default bfloat16)."""
    import torch

    if not mask.is_cuda or not mask.is_contiguous() or mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("mask must be a contiguous bool or uint8 device tensor")
    if out is None:
        out = torch.empty(mask.shape, dtype=out_dtype or torch.bfloat16, device=mask.device)
    _check_output("out", out, tuple(mask.shape), (torch.float16, torch.bfloat16), mask.device)
    _check(load().sdpa_mask_convert(_ptr(mask), _ptr(out), mask.numel(), _dtype_code(out), _stream_handle(stream)))
    return out


def hbm_read_probe(data, *, sink=None, stream=None):
    """Measurement helper (``sdpa_hbm_read_probe``): reads every byte of the
    contiguous device tensor ``data`` once; its time gives the streaming-read
    rate.  ``sink`` is a uint32-compatible device tensor of 2048 elements
    (allocated if None), returned."""
    import torch

    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous device tensor")
    nbytes = data.numel() * data.element_size()
    if nbytes % 16:
        raise ValueError(f"data must hold a multiple of 16 bytes (got {nbytes})")
    if sink is None:
        sink = torch.empty(2048, dtype=torch.int32, device=data.device)
    _require(sink.is_cuda and sink.is_contiguous() and sink.element_size() == 4 and sink.numel() >= 2048,
             "sink must be a contiguous 4-byte device tensor of at least 2048 elements")
    _check(load().sdpa_hbm_read_probe(_ptr(data), nbytes, _ptr(sink), _stream_handle(stream)))
    return sink


def prefill_masked(q, k, v, mask, *, scale=None, causal=False, out=None, lse=None, stream=None):
    """O = softmax(Q K^T * scale + mask [+ causal]) V (``sdpa_prefill_masked_fwd``).

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] fp16/bf16; ``mask`` an additive mask
    of q's dtype, a [Bm, Hm, Sq, W] view with Bm in {1, B}, Hm in {1, Hq}
    (size-1 dims broadcast) and W >= Sk whose last dim is contiguous; its
    strides must be multiples of 8 elements (pad rows to a multiple of 8 and
    slice them to Sk: ``mask[..., :Sk]`` of a padded tensor qualifies)."""
    import torch

    _check_inputs(("q", "k", "v"), (q, k, v))
    _check_prefill_shapes(q, k, v)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    _require(mask.device == q.device, f"mask is on {mask.device}, q on {q.device}")
    if mask.dim() != 4 or mask.dtype != q.dtype or not mask.is_cuda or mask.stride(-1) != 1:
        raise ValueError("mask must be a 4-D device tensor of q's dtype with a contiguous last dim")
    if mask.shape[0] not in (1, B) or mask.shape[1] not in (1, Hq) or mask.shape[2] != Sq or mask.shape[3] < Sk:
        raise ValueError(f"mask shape {tuple(mask.shape)} does not cover [{B}, {Hq}, {Sq}, {Sk}]")
    sb = 0 if mask.shape[0] == 1 else mask.stride(0)
    sh = 0 if mask.shape[1] == 1 else mask.stride(1)
    _check_output("out", out, (B, Sq, Hq, v.shape[-1]), (q.dtype,), q.device)
    _check_output("lse", lse, (B, Hq, Sq), (torch.float32,), q.device)
    if out is None:
        out = torch.empty(B, Sq, Hq, v.shape[-1], dtype=q.dtype, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    pr = make_problem(batch=B, q_len=Sq, kv_len=Sk, head_q=Hq, head_kv=Hkv, d_qk=D, d_v=v.shape[-1],
                      in_dtype=_dtype_code(q), out_dtype=_dtype_code(out), causal=causal, scale=scale)
    _check(load().sdpa_prefill_masked_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), sb, sh,
                                          mask.stride(2), _ptr(out), _ptr(lse), _stream_handle(stream)))
    return out
