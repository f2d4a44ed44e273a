"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding and
compare with the CPU oracle on the same seeded inputs.

Tolerances (fixed by the library's accuracy contract):
  bf16 forward:   O max-abs <= 2e-2 and rel-L2 <= 1e-2
  bf16 gradients: dQ, dK, dV rel-L2 <= 3e-2
  fp32:           O, dQ, dK, dV max-abs <= 1e-4
  LSE (diagnostic): abs <= 1e-3 (bf16) / 1e-5 (fp32)
  fp8 forward (E4M3 inputs; P rounded to E4M3 before P V, relative error <= 2^-4 per
  element, about 2^-4/sqrt(3) ~ 3.6e-2 in relative L2 of O): O rel-L2 <= 5e-2 and
  max-abs <= 1e-1 against the exact attention of the real inputs; LSE abs <= 1e-3
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {
    "bf16": {"o_abs": 2e-2, "o_rel": 1e-2, "g_rel": 3e-2, "lse_abs": 1e-3},
    "fp32": {"abs": 1e-4, "lse_abs": 1e-5},
    "fp8": {"o_abs": 1e-1, "o_rel": 5e-2, "lse_abs": 1e-3},
}


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def check(name: str, dtype: str, got, ref, kind: str):
    """kind: 'o', 'g' (gradient) or 'lse'. Raises AssertionError with the figures."""
    got = f64(got) if isinstance(got, torch.Tensor) else got
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    ma, rel = errors(got, ref)
    msg = f"{name} ({dtype}): max-abs {ma:.3e} rel-L2 {rel:.3e}"
    print(msg, flush=True)
    if kind == "lse":
        assert ma <= TOL[dtype]["lse_abs"], msg
    elif dtype == "fp32":
        assert ma <= TOL["fp32"]["abs"], msg
    elif dtype == "fp8":
        assert ma <= TOL["fp8"]["o_abs"] and rel <= TOL["fp8"]["o_rel"], msg
    elif kind == "o":
        assert ma <= TOL["bf16"]["o_abs"] and rel <= TOL["bf16"]["o_rel"], msg
    else:
        assert rel <= TOL["bf16"]["g_rel"], msg


def run_gpu(inp, causal: bool, scale: float, dev="cuda"):
    import exact_io_aware_attention_amd as fa
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.do))
    cu = inp.cu_seqlens.to(dev) if inp.cu_seqlens is not None else None
    ms = inp.max_seqlen if cu is not None else None
    o, lse = fa.forward(q, k, v, causal=causal, softmax_scale=scale, cu_seqlens=cu, max_seqlen=ms)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, softmax_scale=scale,
                             cu_seqlens=cu, max_seqlen=ms)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def full_parity(inp, causal: bool, scale: float, dtype: str, label: str):
    """Whole-tensor comparison (small problems)."""
    o, lse, dq, dk, dv = run_gpu(inp, causal, scale)
    cu = inp.cu_seqlens.numpy() if inp.cu_seqlens is not None else None
    o_ref, lse_ref = oracle.forward(inp.q, inp.k, inp.v, scale, causal, cu_seqlens=cu)
    dq_r, dk_r, dv_r = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal, cu_seqlens=cu)
    check(f"{label} O", dtype, o, o_ref, "o")
    check(f"{label} LSE", dtype, lse, lse_ref, "lse")
    check(f"{label} dQ", dtype, dq, dq_r, "g")
    check(f"{label} dK", dtype, dk, dk_r, "g")
    check(f"{label} dV", dtype, dv, dv_r, "g")
    return o, lse, dq, dk, dv
