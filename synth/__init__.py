"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no attention arithmetic: it only draws i.i.d. N(0,1) numbers from
numpy's PCG64 generator and rounds them to bfloat16 bit patterns (round to nearest,
ties to even), so that the HIP path and the CPU oracle read identical bits.

The workloads mirror the shapes the pages discuss: per-head Q, K, V of shape [N, d]
with d = 64 or 128 ("Attention fundamentals", §2.1 and the §2.2 table), sequence lengths
from 1K to 16K ("FlashAttention: Fast and Memory-Efficient Exact Attention with
IO-Awareness", Experimental setup), and a grouped-query KV cache for single-token decode
("FlashAttention optimisation: breaking the attention memory bottleneck", §4.2.2 and §5.3).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "normal_f32", "Workload", "WORKLOADS",
    "make_prefill", "make_decode", "make_varlen", "default_scale",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite (normal draws), so no NaN special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def default_scale(d: int) -> float:
    """1/sqrt(d) as the float32 value both sides use."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int          # query length (1 for decode)
    L: int          # key length
    d: int
    dtype: str      # "bf16" or "f32"
    causal: bool
    qk_mult: float  # exact power-of-two multiplier on Q and K
    seed: int
    kind: str       # "fwd", "fwdbwd" or "decode"


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 256, 64, "f32", False, 1.0, 1001, "fwd"),
    "prefill": Workload("prefill", 4, 16, 16, 1024, 1024, 64, "bf16", True, 1.0, 1002, "fwd"),
    "long4k": Workload("long4k", 1, 32, 32, 4096, 4096, 128, "bf16", True, 2.0, 1003, "fwd"),
    "long8k": Workload("long8k", 1, 32, 32, 8192, 8192, 128, "bf16", True, 2.0, 1003, "fwd"),
    "long16k": Workload("long16k", 1, 32, 32, 16384, 16384, 128, "bf16", True, 2.0, 1003, "fwd"),
    "train": Workload("train", 2, 16, 16, 4096, 4096, 128, "bf16", True, 1.0, 1004, "fwdbwd"),
    "decode": Workload("decode", 64, 32, 8, 1, 8192, 128, "bf16", False, 1.0, 1005, "decode"),
}


def _as_io(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_prefill(B, Hq, Hkv, N, d, dtype="bf16", seed=0, qk_mult=1.0, with_dout=False, L=None):
    """Q [B,Hq,N,d], K/V [B,Hkv,L,d] (L defaults to N), optional dO [B,Hq,N,d].

    Drawn in the order Q, K, V, dO from one PCG64 stream.  For bf16 the arrays are uint16
    bit patterns, else float32.  qk_mult must be a power of two so that scaling is exact.
    """
    L = N if L is None else L
    rng = np.random.default_rng(seed)
    q = normal_f32(rng, (B, Hq, N, d))
    k = normal_f32(rng, (B, Hkv, L, d))
    v = normal_f32(rng, (B, Hkv, L, d))
    out = {}
    if qk_mult != 1.0:
        assert math.log2(qk_mult).is_integer()
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    out["q"], out["k"], out["v"] = _as_io(q, dtype), _as_io(k, dtype), _as_io(v, dtype)
    del q, k, v
    if with_dout:
        out["dout"] = _as_io(normal_f32(rng, (B, Hq, N, d)), dtype)
    return out


def make_decode(B, Hq, Hkv, L, d, seed=0, dtype="bf16"):
    """Q [B,Hq,d] (one token per sequence) and K/V caches [B,Hkv,L,d], drawn Q, K, V.

    Large caches are drawn and rounded in slices of one (b) to bound host memory.
    """
    rng = np.random.default_rng(seed)
    q = _as_io(normal_f32(rng, (B, Hq, d)), dtype)
    io_dt = np.uint16 if dtype == "bf16" else np.float32
    caches = []
    for _ in range(2):
        c = np.empty((B, Hkv, L, d), dtype=io_dt)
        for b in range(B):
            c[b] = _as_io(normal_f32(rng, (Hkv, L, d)), dtype)
        caches.append(c)
    return {"q": q, "k": caches[0], "v": caches[1]}


def make_varlen(lens_q, lens_k, Hq, Hkv, d, dtype="bf16", seed=0, qk_mult=1.0, with_dout=False):
    """Packed variable-length inputs: Q [Hq,total_q,d], K/V [Hkv,total_k,d] with sequence b
    at rows cu_q[b]..cu_q[b+1]-1 (cu_k likewise); cu_q, cu_k are int32 [B+1] running sums of
    the lengths; optional dO [Hq,total_q,d].  Drawn Q, K, V, dO from one PCG64 stream,
    rounded as in make_prefill.
    """
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = normal_f32(rng, (Hq, int(cu_q[-1]), d))
    k = normal_f32(rng, (Hkv, int(cu_k[-1]), d))
    v = normal_f32(rng, (Hkv, int(cu_k[-1]), d))
    if qk_mult != 1.0:
        assert math.log2(qk_mult).is_integer()
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    out = {"q": _as_io(q, dtype), "k": _as_io(k, dtype), "v": _as_io(v, dtype), "cu_q": cu_q, "cu_k": cu_k}
    if with_dout:
        out["dout"] = _as_io(normal_f32(rng, (Hq, int(cu_q[-1]), d)), dtype)
    return out
