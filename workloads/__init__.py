"""Seeded synthetic inputs for exact attention: shapes, dtypes, seeds, packing.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds no attention arithmetic: it only draws random numbers, rounds
them to the storage dtype and lays them out. The oracle and the HIP library each
compute everything else on their own.

Workloads (the five attention shapes the library is measured and checked on):

* ``c1``  single head, B=1, H=1, N=128, d=64, fp32, non-causal, scale 1/sqrt(64)
* ``c2``  BERT/GPT-2-shaped, B=8, H=16, N=2048, d=64, bf16, non-causal
* ``c3``  Llama-shaped, B=4, H=32, N=4096, d=128, bf16, causal, values N(0,1)*0.5
* ``c4``  long context, B=1, H=8, N=65536, d=64, bf16, non-causal
* ``c5``  packed variable length: 16384 tokens, lengths uniform in [128, 2048]
          (last one truncated to fit), H=32, d=128, bf16, causal per sequence

Each is a synthetic stand-in for the transformer training workloads the
FlashAttention pages speak of (BERT, GPT-2 and Llama training, long contexts and
sequence packing). Where a shape leaves the softmax scale open it is 1/sqrt(d).

Layout: (batch, seqlen, heads, head_dim), head_dim innermost; packed batches are
(total_tokens, heads, head_dim) with ``cu_seqlens`` int32 [batch + 1].
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "get", "make_inputs", "varlen_lengths",
    "cu_seqlens_from_lengths", "sample_rows", "Inputs",
    "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int              # number of sequences (for packed: filled in from the lengths)
    heads: int
    seqlen: int             # N (for packed: the maximum length the lengths may take)
    head_dim: int
    dtype: str              # "bf16" or "fp32"
    causal: bool
    std: float              # inputs are iid N(0, 1) * std
    seed: int
    varlen_total: int = 0   # > 0: packed variable-length batch of this many tokens
    varlen_lo: int = 0
    varlen_hi: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def varlen(self) -> bool:
        return self.varlen_total > 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 128, 64, "fp32", False, 1.0, 1001,
                   description="single head exact attention, fp32"),
    "c2": Workload("c2", 8, 16, 2048, 64, "bf16", False, 1.0, 1002,
                   description="BERT/GPT-2-shaped attention"),
    "c3": Workload("c3", 4, 32, 4096, 128, "bf16", True, 0.5, 1003,
                   description="Llama-shaped causal attention"),
    "c4": Workload("c4", 1, 8, 65536, 64, "bf16", False, 1.0, 1004,
                   description="long-context attention"),
    "c5": Workload("c5", 0, 32, 2048, 128, "bf16", True, 1.0, 1005,
                   varlen_total=16384, varlen_lo=128, varlen_hi=2048,
                   description="packed variable-length causal attention"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def varlen_lengths(seed: int, total: int, lo: int, hi: int) -> List[int]:
    """Sequence lengths drawn uniformly from [lo, hi] (inclusive) until they reach
    ``total`` tokens; the last one is cut so the lengths sum to exactly ``total``
    (it may come out shorter than ``lo``, which is kept as a ragged case)."""
    rng = np.random.default_rng(seed)
    lengths: List[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lengths.append(n)
        acc += n
    return lengths


def cu_seqlens_from_lengths(lengths: List[int]) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def sample_rows(seed: int, n: int, count: int) -> np.ndarray:
    """``count`` distinct row indices out of ``n``, sorted (seeded)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(count, n), replace=False)).astype(np.int64)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]   # int32 [batch+1] (CPU) or None
    lengths: Optional[List[int]]
    batch: int
    seqlen: int                          # N, or the longest sequence of a packed batch
    total_tokens: int

    @property
    def max_seqlen(self) -> int:
        return self.seqlen


def _randn(shape, seed: int, std: float, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)   # round-to-nearest-even to the storage dtype


def make_inputs(w: Workload, seed: Optional[int] = None, *, batch: Optional[int] = None,
                seqlen: Optional[int] = None, heads: Optional[int] = None,
                lengths: Optional[List[int]] = None) -> Inputs:
    """Seeded Q, K, V, dO on the CPU in the workload's storage dtype.

    Tensor ``i`` (0=Q, 1=K, 2=V, 3=dO) comes from ``torch.Generator`` seeded with
    ``seed + i``. ``batch``/``seqlen``/``heads``/``lengths`` override the workload's
    shape (used for small parity cases with the same recipe)."""
    seed = w.seed if seed is None else seed
    H = w.heads if heads is None else heads
    d = w.head_dim
    dt = w.torch_dtype
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(seed, w.varlen_total, w.varlen_lo, w.varlen_hi)
        cu = cu_seqlens_from_lengths(lengths)
        T = int(cu[-1])
        shape = (T, H, d)
        B = len(lengths)
        N = max(lengths) if lengths else 0
    else:
        B = w.batch if batch is None else batch
        N = w.seqlen if seqlen is None else seqlen
        shape = (B, N, H, d)
        cu = None
        T = B * N
    q, k, v, do = (_randn(shape, seed + i, w.std, dt) for i in range(4))
    return Inputs(w, q, k, v, do, cu, list(lengths) if lengths is not None else None, B, N, T)


# ---------------------------------------------------------------- decoding

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """seqlen_q new queries against a cache of seqlen_k keys and values (the last
    seqlen_q positions of the sequence)."""
    name: str
    batch: int
    heads: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool
    std: float
    seed: int
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# Synthetic stand-ins for generation with a long key cache (the pages cite faster
# inference without a shape): one new token, and a 16-token chunk (speculative or
# chunked decoding), against 16384 cached positions, Llama-shaped heads.
DECODE_WORKLOADS = {
    "d1": DecodeWorkload("d1", 8, 32, 1, 16384, 128, True, 1.0, 2001,
                         description="decode: 1 query against a 16384-key cache"),
    "d2": DecodeWorkload("d2", 8, 32, 16, 16384, 128, True, 1.0, 2002,
                         description="decode: 16 queries against a 16384-key cache"),
}


def make_decode_inputs(w: DecodeWorkload, seed: Optional[int] = None, *, batch: Optional[int] = None,
                       seqlen_q: Optional[int] = None, seqlen_k: Optional[int] = None,
                       heads: Optional[int] = None, head_dim: Optional[int] = None):
    """Seeded bf16 Q (B, Nq, H, d), K and V (B, Nk, H, d) on the CPU, drawn like
    ``make_inputs`` (tensor i from a generator seeded seed + i)."""
    seed = w.seed if seed is None else seed
    B = w.batch if batch is None else batch
    Nq = w.seqlen_q if seqlen_q is None else seqlen_q
    Nk = w.seqlen_k if seqlen_k is None else seqlen_k
    H = w.heads if heads is None else heads
    d = w.head_dim if head_dim is None else head_dim
    q = _randn((B, Nq, H, d), seed, w.std, torch.bfloat16)
    k = _randn((B, Nk, H, d), seed + 1, w.std, torch.bfloat16)
    v = _randn((B, Nk, H, d), seed + 2, w.std, torch.bfloat16)
    return q, k, v


# ---------------------------------------------------------------- 8-bit inputs

@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """Forward pass on OCP FP8 E4M3 inputs with per-tensor descale factors."""
    name: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    causal: bool
    std: float
    seed: int
    descale_q: float = 1.0
    descale_k: float = 1.0
    descale_v: float = 1.0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The Llama-shaped training workload with its inputs stored in 8 bits (the pages name
# 8-bit floating point for FlashAttention-3 without a workload).
FP8_WORKLOADS = {
    "f1": Fp8Workload("f1", 4, 32, 4096, 128, True, 1.0, 3001,
                      description="c3 shape, E4M3 Q, K, V"),
}


def make_fp8_inputs(w: Fp8Workload, seed: Optional[int] = None, *, batch: Optional[int] = None,
                    seqlen: Optional[int] = None, heads: Optional[int] = None, head_dim: Optional[int] = None):
    """Seeded uint8 E4M3 codes q8, k8, v8 (B, N, H, d) on the CPU: iid normal values of
    standard deviation w.std, each divided by its tensor's descale, rounded to E4M3 by
    torch's float8_e4m3fn conversion (tensor i from a generator seeded seed + i)."""
    seed = w.seed if seed is None else seed
    B = w.batch if batch is None else batch
    N = w.seqlen if seqlen is None else seqlen
    H = w.heads if heads is None else heads
    d = w.head_dim if head_dim is None else head_dim
    out = []
    for i, ds in enumerate((w.descale_q, w.descale_k, w.descale_v)):
        g = torch.Generator().manual_seed(seed + i)
        x = torch.randn((B, N, H, d), generator=g, dtype=torch.float32) * (w.std / ds)
        out.append(x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous())
    return tuple(out)


def make_device_tensors(shape, count: int, seed: int, std: float, dtype: torch.dtype,
                        device="cuda") -> tuple:
    """`count` seeded iid normal tensors of one shape generated on the device (for
    inputs of several GiB, where host generation is slow): tensor i is torch.randn from
    a device generator seeded seed + i, times std, rounded to `dtype` (RNE; for
    torch.uint8 the values are rounded to E4M3 by torch's float8_e4m3fn conversion and
    returned as their codes). Built 2^26 elements at a time, so the fp32 temporary stays
    small."""
    n = math.prod(shape)
    chunk = 1 << 26
    out = []
    for i in range(count):
        g = torch.Generator(device=device)
        g.manual_seed(seed + i)
        t = torch.empty(n, device=device, dtype=dtype)
        for a in range(0, n, chunk):
            x = torch.randn(min(chunk, n - a), generator=g, device=device, dtype=torch.float32)
            if std != 1.0:
                x.mul_(std)
            t[a:a + x.numel()] = x.to(torch.float8_e4m3fn).view(torch.uint8) if dtype == torch.uint8 else x.to(dtype)
        out.append(t.view(shape))
    return tuple(out)
