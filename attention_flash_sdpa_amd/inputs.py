"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws i.i.d. N(0,1) values
and casts them to the storage dtype.  Both the HIP path (through the tests and
the benchmark) and the fp64 CPU oracle consume exactly these tensors.

Recipe (the pages run on no dataset; "xe2-sdp-kernels", section "Performance
testing", asks for random non-zero inputs):
  * values are drawn in fp32 from a CPU ``torch.Generator`` seeded with the
    workload's seed, in the order Q, K, V;
  * bf16 / fp16 storage: cast with round-to-nearest-even;
  * fp8 storage (OCP e4m3fn, largest finite 448): per-tensor scale
    sigma = amax(|x|) / 448, x_q = e4m3fn(RNE(clamp(x / sigma, +-448))); the
    dequantised value is x_q * sigma;
  * rotating K/V sets for the memory-bound decode workload use seed
    ``seed + 100 * set_index`` (the same page asks for N_BUF = 4 rotating
    buffer sets for memory-bound kernels).
"""
from __future__ import annotations

import dataclasses
import math

import torch

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention problem (layouts: Q [B,Sq,Hq,D], K/V [B,Sk,Hkv,D|Dv])."""

    name: str
    batch: int
    head_q: int
    head_kv: int
    q_len: int
    kv_len: int
    d_qk: int
    d_v: int
    dtype: str            # storage dtype of Q/K/V: "f16", "bf16", "fp8_e4m3"
    out_dtype: str        # "f16" or "bf16"
    causal: bool
    seed: int
    decode: bool = False  # q_len == 1 through the split-KV decode entry point
    kv_sets: int = 1      # rotating K/V buffer sets for timing

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def valid_pairs(self) -> int:
        """Query-key pairs that are visible (bottom-right causal rule)."""
        if not self.causal:
            return self.q_len * self.kv_len
        off = self.kv_len - self.q_len
        return sum(max(0, min(self.kv_len, i + off + 1)) for i in range(self.q_len))

    def flops(self) -> int:
        """Algorithmic FLOP: 2*(D + Dv) per visible pair, per query head."""
        return 2 * (self.d_qk + self.d_v) * self.valid_pairs() * self.head_q * self.batch

    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once and O written once."""
        el = 1 if self.dtype == "fp8_e4m3" else 2
        el_out = 2
        q = self.batch * self.q_len * self.head_q * self.d_qk * el
        k = self.batch * self.kv_len * self.head_kv * self.d_qk * el
        v = self.batch * self.kv_len * self.head_kv * self.d_v * el
        o = self.batch * self.q_len * self.head_q * self.d_v * el_out
        return q + k + v + o


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f16_128", 1, 1, 1, 128, 128, 64, 64, "f16", "f16", False, 1001),
        Workload("gqa_causal_prefill_bf16", 1, 32, 8, 512, 1024, 128, 128, "bf16", "bf16", True, 1002),
        Workload("unaligned_full_bf16", 2, 28, 4, 1001, 1023, 128, 128, "bf16", "bf16", False, 1003),
        Workload("tiny_causal_bf16", 2, 28, 4, 7, 5, 128, 128, "bf16", "bf16", True, 1013),
        Workload("splitkv_decode_bf16", 16, 32, 8, 1, 8192, 128, 128, "bf16", "bf16", False, 1004,
                 decode=True, kv_sets=4),
        Workload("mla_fp8_causal_prefill", 1, 128, 128, 4096, 4096, 192, 128, "fp8_e4m3", "bf16", True, 1005),
    ]
}

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def quantize_fp8(x: torch.Tensor):
    """Per-tensor e4m3fn quantisation; returns (x_q, sigma) with x ~= x_q * sigma."""
    amax = float(x.abs().max())
    sigma = amax / FP8_MAX if amax > 0 else 1.0
    xq = (x / sigma).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return xq, sigma


def cast(x: torch.Tensor, dtype: str):
    """Casts fp32 draws to the storage dtype; returns (tensor, descale)."""
    if dtype == "fp8_e4m3":
        return quantize_fp8(x)
    return x.to(_TORCH_DTYPES[dtype]), 1.0


def draw(shape, gen: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def make_qkv(w: Workload, *, seed: int | None = None, kv_set: int = 0, q_len: int | None = None,
             kv_len: int | None = None):
    """Draws (q, k, v, descales) on the CPU for workload ``w``.

    ``kv_set`` selects a rotating K/V set (seed + 100*kv_set); Q always comes
    from the base seed.  ``q_len`` / ``kv_len`` override the workload's lengths
    (used for reduced-size parity cases).
    """
    seed = w.seed if seed is None else seed
    sq = w.q_len if q_len is None else q_len
    sk = w.kv_len if kv_len is None else kv_len
    g = torch.Generator().manual_seed(seed)
    q32 = draw((w.batch, sq, w.head_q, w.d_qk), g)
    if kv_set:
        g = torch.Generator().manual_seed(seed + 100 * kv_set)
        draw((w.batch, sq, w.head_q, w.d_qk), g)      # keep the Q, K, V draw order
    k32 = draw((w.batch, sk, w.head_kv, w.d_qk), g)
    v32 = draw((w.batch, sk, w.head_kv, w.d_v), g)
    q, sq_ = cast(q32, w.dtype)
    del q32
    k, sk_ = cast(k32, w.dtype)
    del k32
    v, sv_ = cast(v32, w.dtype)
    return q, k, v, (sq_, sk_, sv_)


def paginate(k: torch.Tensor, v: torch.Tensor, page_size: int, *, seed: int, spare_pages: int = 0,
             fill: float = float("nan")):
    """Scatters dense caches k, v [B, Sk, Hkv, D|Dv] into page pools
    [B * P + spare_pages, page_size, Hkv, D|Dv] (P = ceil(Sk / page_size)) in a
    seeded random physical order.  Returns (k_pool, v_pool, page_table) with
    page_table int32 [B, P]: logical page p of sequence b is pool page
    page_table[b, p].  Slots past Sk and the spare pages hold ``fill`` (NaN by
    default, so a read of a slot no sequence owns shows in the output)."""
    B, Sk, Hkv, D = k.shape
    Dv = v.shape[-1]
    P = -(-Sk // page_size)
    n = B * P + spare_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed))[:B * P]
    table = perm.reshape(B, P).to(torch.int32)
    kp = torch.full((n, page_size, Hkv, D), fill, dtype=torch.float32).to(k.dtype)
    vp = torch.full((n, page_size, Hkv, Dv), fill, dtype=torch.float32).to(v.dtype)
    for b in range(B):
        for p in range(P):
            lo, hi = p * page_size, min(Sk, (p + 1) * page_size)
            kp[table[b, p], :hi - lo] = k[b, lo:hi]
            vp[table[b, p], :hi - lo] = v[b, lo:hi]
    return kp, vp, table


def length_mix(batch: int, kv_len: int, *, seed: int) -> torch.Tensor:
    """Seeded per-sequence key counts in [0, kv_len] for variable-length
    decode: the first sequences take the edge values 0, 1 and kv_len, the rest
    are uniform draws (int32 [batch])."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(0, kv_len + 1, (batch,), generator=g)
    edges = [0, 1, kv_len][:batch]
    lens[:len(edges)] = torch.tensor(edges)
    return lens.to(torch.int32)
