"""FP8 (E4M3) inputs for the forward pass: decoding and the exact attention of the
decoded values, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY: called by tests and the benchmark's CPU-baseline leg, never
by the library.

Source: [SA] "FlashAttention-2 (PT)" (Systems analysis wiki), section "Comparação com
versões subsequentes" / "FlashAttention-3": the later version adds 8-bit floating-point
computation for more speed. The pages fix no format, scaling or accuracy; readings:

* r16 the 8-bit format is OCP FP8 E4M3 ("E4M3FN": 1 sign bit, 4 exponent bits with bias
      7, 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN, largest finite
      magnitude 448); each of Q, K, V carries one fp32 descale factor per tensor, the
      real value being descale * decoded; O is bf16 and LSE fp32 as in the bf16 path.
      The target is the exact attention of the real (decoded, descaled) inputs, which is
      what ``forward_fp8`` computes; the GPU kernel also rounds P to E4M3 before P V, and
      its accuracy is judged against this exact result.

Parity pinned: ``e4m3_decode`` (spec constants, grid and ordering properties) and
``forward_fp8`` (closed forms and hand-decoded brute force) in tests/test_oracle_fp8.py.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import forward

Array = np.ndarray


def e4m3_decode(codes) -> Array:
    """fp64 values of OCP E4M3 codes (uint8 array of any shape); NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, v)


def forward_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, scale: float,
                causal: bool) -> Tuple[Array, Array]:
    """O and LSE of attention on the real inputs descale * decode(code); q8, k8, v8 are
    (B, N, H, d) uint8 codes; O (B, N, H, d) and LSE (B, H, N) in fp64."""
    q = e4m3_decode(q8) * float(descale_q)
    k = e4m3_decode(k8) * float(descale_k)
    v = e4m3_decode(v8) * float(descale_v)
    return forward(q, k, v, scale, causal)
