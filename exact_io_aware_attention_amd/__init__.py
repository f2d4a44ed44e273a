"""exact_io_aware_attention_amd: exact IO-aware attention on AMD MI355X (gfx950).

A thin Python binding over ``libfa.so``, whose C ABI is declared in ``include/fa.h``.
The raw entry points keep the C names and take integer device pointers:

    fa_fwd, fa_bwd, fa_bwd_atomic, fa_bwd_noalloc, fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dq_stats,
    fa_bwd_workspace_bytes, fa_bwd_atomic_workspace_bytes, fa_fwd_decode, fa_fwd_decode_workspace_bytes,
    fa_fwd_fp8, fa_strerror

``forward``, ``backward``, ``decode`` and ``forward_fp8`` marshal torch tensors (device memory and the current
stream) into those calls; every step of the computation runs in the HIP kernels.
There is no fallback: if ``libfa.so`` is missing or fails to load, every call raises.
Build it with ``python -m exact_io_aware_attention_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_SCRATCH",
    "FA_BWD_NOALLOC_MAX_SCRATCH", "fa_bwd_noalloc",
    "FA_DTYPE_BF16", "FA_DTYPE_FP32", "FAError", "library_path", "load_library",
    "fa_fwd", "fa_bwd", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_workspace_bytes",
    "fa_bwd_atomic", "fa_bwd_atomic_workspace_bytes",
    "fa_strerror", "forward", "backward", "decode", "fa_fwd_decode", "fa_fwd_decode_workspace_bytes",
    "fa_fwd_fp8", "forward_fp8", "fa_device_info", "fa_ubench_mfma_bf16", "fa_ubench_mfma_fp8", "fa_ubench_valu", "fa_ubench_lds", "fa_ubench_copy",
    "fa_ubench_mfma_valu", "fa_ubench_mfma_mix",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
FA_BWD_NOALLOC_MAX_SCRATCH = (16 << 20) + 256   # bytes of fa_bwd_noalloc's fixed device array (include/fa.h)
FA_DTYPE_BF16, FA_DTYPE_FP32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {fa_strerror(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load_library() -> ctypes.CDLL:
    """Load libfa.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m exact_io_aware_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, i32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                           i32, i32, i32, i32, f32, i32, vp, i32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_atomic.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                  i32, i32, i32, i32, f32, i32, vp, i32, i32, vp]
    lib.fa_bwd_atomic.restype = i32
    lib.fa_bwd_atomic_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_bwd_atomic_workspace_bytes.restype = sz
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, i32, i32,
                                   vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i32, i32, i32, i32, f32, vp, i32, i32, vp]
    lib.fa_bwd_preprocess.restype = i32
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, vp, i32, i32, i32, i32, f32, i32, vp, i32, i32, vp]
    lib.fa_bwd_dkdv.restype = i32
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, i32, i32, i32, i32, f32, i32, vp, i32, i32, vp]
    lib.fa_bwd_dq.restype = i32
    lib.fa_bwd_dq_stats.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i32, i32, i32, i32, f32, i32, vp, i32, i32,
                                    vp]
    lib.fa_bwd_dq_stats.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, i32, vp]
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, f32, f32, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_fwd_decode.restype = i32
    lib.fa_fwd_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_decode_workspace_bytes.restype = sz
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_device_info.argtypes = [i32, ip, ip, ip, ctypes.c_char_p, i32]
    lib.fa_device_info.restype = i32
    lib.fa_ubench_mfma_bf16.argtypes = [vp, i32, i32, vp]
    lib.fa_ubench_mfma_bf16.restype = i32
    lib.fa_ubench_mfma_fp8.argtypes = [vp, i32, i32, vp]
    lib.fa_ubench_mfma_fp8.restype = i32
    lib.fa_ubench_valu.argtypes = [vp, i32, i32, i32, vp]
    lib.fa_ubench_valu.restype = i32
    lib.fa_ubench_lds.argtypes = [vp, i32, i32, i32, vp]
    lib.fa_ubench_lds.restype = i32
    lib.fa_ubench_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.fa_ubench_copy.restype = i32
    lib.fa_ubench_mfma_valu.argtypes = [vp, i32, i32, i32, i32, i32, vp]
    lib.fa_ubench_mfma_valu.restype = i32
    lib.fa_ubench_mfma_mix.argtypes = [vp, i32, i32, i32, vp]
    lib.fa_ubench_mfma_mix.restype = i32
    _LIB = lib
    return lib


# ---------------------------------------------------------------- raw C entry points

def fa_fwd(q: int, k: int, v: int, o: int, lse: int, batch: int, heads: int, seqlen: int,
           head_dim: int, softmax_scale: float, causal: int, cu_seqlens: Optional[int],
           total_tokens: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_fwd(q, k, v, o, lse, batch, heads, seqlen, head_dim, softmax_scale,
                                 int(causal), cu_seqlens, total_tokens, dtype, stream)


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
           workspace: int, workspace_bytes: int, batch: int, heads: int, seqlen: int, head_dim: int,
           softmax_scale: float, causal: int, cu_seqlens: Optional[int], total_tokens: int,
           dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                                 batch, heads, seqlen, head_dim, softmax_scale, int(causal),
                                 cu_seqlens, total_tokens, dtype, stream)


def fa_bwd_atomic(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
                  workspace: int, workspace_bytes: int, batch: int, heads: int, seqlen: int, head_dim: int,
                  softmax_scale: float, causal: int, cu_seqlens: Optional[int], total_tokens: int,
                  dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd_atomic(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                                        batch, heads, seqlen, head_dim, softmax_scale, int(causal),
                                        cu_seqlens, total_tokens, dtype, stream)


def fa_bwd_atomic_workspace_bytes(batch: int, heads: int, seqlen: int, head_dim: int, varlen: int,
                                  total_tokens: int) -> int:
    return load_library().fa_bwd_atomic_workspace_bytes(batch, heads, seqlen, head_dim, int(varlen), total_tokens)


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, batch: int,
                   heads: int, seqlen: int, head_dim: int, softmax_scale: float, causal: int,
                   cu_seqlens: Optional[int], total_tokens: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, seqlen, head_dim,
                                         softmax_scale, int(causal), cu_seqlens, total_tokens, dtype, stream)


def fa_bwd_preprocess(o: int, dout: int, lse: int, workspace: int, workspace_bytes: int, batch: int, heads: int,
                      seqlen: int, head_dim: int, softmax_scale: float, cu_seqlens: Optional[int],
                      total_tokens: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd_preprocess(o, dout, lse, workspace, workspace_bytes, batch, heads, seqlen,
                                            head_dim, softmax_scale, cu_seqlens, total_tokens, dtype, stream)


def fa_bwd_dkdv(q: int, k: int, v: int, dout: int, lse: int, workspace: int, workspace_bytes: int,
                dk: int, dv: int, batch: int, heads: int, seqlen: int, head_dim: int, softmax_scale: float,
                causal: int, cu_seqlens: Optional[int], total_tokens: int, dtype: int,
                stream: Optional[int]) -> int:
    return load_library().fa_bwd_dkdv(q, k, v, dout, lse, workspace, workspace_bytes, dk, dv, batch, heads,
                                      seqlen, head_dim, softmax_scale, int(causal), cu_seqlens, total_tokens,
                                      dtype, stream)


def fa_bwd_dq(q: int, k: int, v: int, dout: int, lse: int, workspace: int, workspace_bytes: int, dq: int,
              batch: int, heads: int, seqlen: int, head_dim: int, softmax_scale: float, causal: int,
              cu_seqlens: Optional[int], total_tokens: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd_dq(q, k, v, dout, lse, workspace, workspace_bytes, dq, batch, heads, seqlen,
                                    head_dim, softmax_scale, int(causal), cu_seqlens, total_tokens, dtype,
                                    stream)


def fa_bwd_dq_stats(q: int, k: int, v: int, o: int, dout: int, lse: int, workspace: int, workspace_bytes: int,
                    dq: int, batch: int, heads: int, seqlen: int, head_dim: int, softmax_scale: float, causal: int,
                    cu_seqlens: Optional[int], total_tokens: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_bwd_dq_stats(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, batch, heads,
                                          seqlen, head_dim, softmax_scale, int(causal), cu_seqlens, total_tokens,
                                          dtype, stream)


def fa_bwd_workspace_bytes(batch: int, heads: int, seqlen: int, head_dim: int, varlen: int,
                           total_tokens: int) -> int:
    return load_library().fa_bwd_workspace_bytes(batch, heads, seqlen, head_dim, int(varlen), total_tokens)


def fa_fwd_fp8(q: int, k: int, v: int, o: int, lse: int, batch: int, heads: int, seqlen: int, head_dim: int,
               softmax_scale: float, descale_q: float, descale_k: float, descale_v: float, causal: int,
               stream: Optional[int]) -> int:
    return load_library().fa_fwd_fp8(q, k, v, o, lse, batch, heads, seqlen, head_dim, softmax_scale, descale_q,
                                     descale_k, descale_v, int(causal), stream)


def fa_fwd_decode(q: int, k: int, v: int, o: int, lse: int, batch: int, heads: int, seqlen_q: int,
                  seqlen_k: int, head_dim: int, softmax_scale: float, causal: int, num_splits: int,
                  workspace: int, workspace_bytes: int, dtype: int, stream: Optional[int]) -> int:
    return load_library().fa_fwd_decode(q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, head_dim,
                                        softmax_scale, int(causal), num_splits, workspace, workspace_bytes,
                                        dtype, stream)


def fa_fwd_decode_workspace_bytes(batch: int, heads: int, seqlen_q: int, seqlen_k: int, head_dim: int,
                                  num_splits: int) -> int:
    return load_library().fa_fwd_decode_workspace_bytes(batch, heads, seqlen_q, seqlen_k, head_dim, num_splits)


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(status).decode()


# ---------------------------------------------------------------- measurement calls (fa_ubench.h)

def fa_device_info(device: int = 0) -> dict:
    """Compute units, maximum engine clock (kHz), L2 bytes and architecture name of a device,
    as the HIP runtime reports them."""
    cu, clk, l2 = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    arch = ctypes.create_string_buffer(64)
    st = load_library().fa_device_info(device, ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(l2), arch, 64)
    if st != FA_OK:
        raise FAError(st, "fa_device_info")
    return {"compute_units": cu.value, "max_clock_khz": clk.value, "l2_bytes": l2.value,
            "arch": arch.value.decode()}


def fa_ubench_mfma_bf16(out: int, blocks: int, iters: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_mfma_bf16(out, blocks, iters, stream)


def fa_ubench_mfma_fp8(out: int, blocks: int, iters: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_mfma_fp8(out, blocks, iters, stream)


def fa_ubench_valu(out: int, blocks: int, iters: int, op: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_valu(out, blocks, iters, op, stream)


def fa_ubench_lds(out: int, blocks: int, iters: int, op: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_lds(out, blocks, iters, op, stream)


def fa_ubench_copy(src: int, dst: int, nbytes: int, blocks: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_copy(src, dst, nbytes, blocks, stream)


def fa_ubench_mfma_valu(out: int, blocks: int, iters: int, nvalu: int, agpr: int, op: int,
                        stream: Optional[int]) -> int:
    return load_library().fa_ubench_mfma_valu(out, blocks, iters, nvalu, agpr, op, stream)


def fa_ubench_mfma_mix(out: int, blocks: int, iters: int, mix: int, stream: Optional[int]) -> int:
    return load_library().fa_ubench_mfma_mix(out, blocks, iters, mix, stream)


# ---------------------------------------------------------------- torch marshalling

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _shape(q, cu_seqlens, max_seqlen):
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("q must be (batch, seqlen, heads, head_dim)")
        B, N, H, d = q.shape
        return B, N, H, d, B * N
    if q.dim() != 3:
        raise ValueError("packed q must be (total_tokens, heads, head_dim)")
    if max_seqlen is None:
        raise ValueError("max_seqlen is required with cu_seqlens")
    T, H, d = q.shape
    return cu_seqlens.numel() - 1, int(max_seqlen), H, d, T


def _check(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if t.device != dev:
            raise ValueError(f"all tensors must be on one device ({dev}), got {t.device}")


def _expect(name: str, t, shape, dtype) -> None:
    """The C entry points take bare pointers sized from q's dimensions, so every other
    tensor is checked here, before any launch, against the shape and dtype it must have."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _lse_shape(B, H, N, T, varlen: bool):
    return (H, T) if varlen else (B, H, N)


def _check_cu(cu_seqlens, B: int, T: int, max_seqlen: int, validate: bool) -> None:
    """cu_seqlens must be int32 [B + 1]. With ``validate`` its values are read back to the
    host (a synchronising copy) and checked, since the kernels trust them: cu[0] = 0,
    non-decreasing, cu[B] = the packed token count, no sequence longer than max_seqlen.
    A larger last entry would send the kernels past the ends of the tensors, a longer
    sequence would leave rows unwritten."""
    import torch
    _expect("cu_seqlens", cu_seqlens, (B + 1,), torch.int32)
    if int(max_seqlen) < 1:
        raise ValueError(f"max_seqlen must be >= 1, got {max_seqlen}")
    if not validate:
        return
    cu = [int(c) for c in cu_seqlens.detach().to("cpu").tolist()]
    if cu[0] != 0:
        raise ValueError(f"cu_seqlens[0] must be 0, got {cu[0]}")
    if cu[-1] != T:
        raise ValueError(f"cu_seqlens[-1] must equal the packed token count {T}, got {cu[-1]}")
    lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
    if min(lens, default=0) < 0:
        raise ValueError("cu_seqlens must be non-decreasing")
    if max(lens, default=0) > int(max_seqlen):
        raise ValueError(f"a sequence of {max(lens)} tokens is longer than max_seqlen = {max_seqlen}")


def _workspace_bytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream):
    import torch
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def forward(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None, cu_seqlens=None,
            max_seqlen: Optional[int] = None, out=None, lse=None, stream=None, check_cu: bool = True) -> Tuple:
    """O and the fp32 natural-log LSE of exact attention (see include/fa.h). For a packed
    batch, ``check_cu`` (default) validates cu_seqlens on a host copy first; pass False to
    skip that synchronising read when the offsets are known to be well formed."""
    import torch
    B, N, H, d, T = _shape(q, cu_seqlens, max_seqlen)
    varlen = cu_seqlens is not None
    _expect("k", k, q.shape, q.dtype)
    _expect("v", v, q.shape, q.dtype)
    if out is not None:
        _expect("out", out, q.shape, q.dtype)
    if lse is not None:
        _expect("lse", lse, _lse_shape(B, H, N, T, varlen), torch.float32)
    if varlen:
        _check_cu(cu_seqlens, B, T, N, check_cu)
    _check(q, k, v, *(t for t in (out, lse, cu_seqlens) if t is not None))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(_lse_shape(B, H, N, T, varlen), device=q.device, dtype=torch.float32)
    cu = cu_seqlens.data_ptr() if varlen else None
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                scale, int(causal), cu, T, _dtype_code(q), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, softmax_scale: Optional[float] = None,
             cu_seqlens=None, max_seqlen: Optional[int] = None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, check_cu: bool = True, deterministic: bool = True) -> Tuple:
    """(dQ, dK, dV) for the upstream gradient ``dout`` (see include/fa.h); ``check_cu`` as
    in ``forward``. ``deterministic=False`` calls fa_bwd_atomic (head_dim 128, bf16: one
    pass with dQ accumulated by fp32 atomics, reproducible up to the last bits of dQ)."""
    import torch
    B, N, H, d, T = _shape(q, cu_seqlens, max_seqlen)
    varlen = cu_seqlens is not None
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _expect(name, t, q.shape, q.dtype)
    _expect("lse", lse, _lse_shape(B, H, N, T, varlen), torch.float32)
    if varlen:
        _check_cu(cu_seqlens, B, T, N, check_cu)
    _check(q, k, v, o, lse, dout, *(t for t in (dq, dk, dv, workspace, cu_seqlens) if t is not None))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    size_fn, call, name = ((fa_bwd_workspace_bytes, fa_bwd, "fa_bwd") if deterministic else
                           (fa_bwd_atomic_workspace_bytes, fa_bwd_atomic, "fa_bwd_atomic"))
    ws_bytes = size_fn(B, H, N, d, int(varlen), T)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    cu = cu_seqlens.data_ptr() if varlen else None
    st = call(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), _workspace_bytes(workspace),
              B, H, N, d, scale, int(causal), cu, T, _dtype_code(q), _stream(stream))
    if st != FA_OK:
        raise FAError(st, name)
    return dq, dk, dv


def decode(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None, num_splits: int = 0,
           out=None, lse=None, workspace=None, stream=None) -> Tuple:
    """O and LSE of seqlen_q (<= 32) new queries against a cache of seqlen_k keys/values
    (see fa_fwd_decode in include/fa.h). q: (batch, seqlen_q, heads, head_dim); k, v:
    (batch, seqlen_k, heads, head_dim); bf16."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be (batch, seqlen, heads, head_dim)")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    _expect("k", k, (B, Nk, H, d), q.dtype)
    _expect("v", v, (B, Nk, H, d), q.dtype)
    if out is not None:
        _expect("out", out, q.shape, q.dtype)
    if lse is not None:
        _expect("lse", lse, (B, H, Nq), torch.float32)
    _check(q, k, v, *(t for t in (out, lse, workspace) if t is not None))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    ws_bytes = fa_fwd_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    st = fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                       scale, int(causal), num_splits, workspace.data_ptr(), _workspace_bytes(workspace),
                       _dtype_code(q),
                       _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_decode")
    return out, lse


def forward_fp8(q8, k8, v8, descale_q: float = 1.0, descale_k: float = 1.0, descale_v: float = 1.0,
                causal: bool = False, softmax_scale: Optional[float] = None, out=None, lse=None,
                stream=None) -> Tuple:
    """O (bf16) and LSE of attention on E4M3 inputs (see fa_fwd_fp8 in include/fa.h).
    q8, k8, v8: (batch, seqlen, heads, head_dim) uint8 tensors of E4M3 codes on the GPU;
    the real inputs are descale * code value."""
    import torch
    if q8.dim() != 4:
        raise ValueError("q8 must be (batch, seqlen, heads, head_dim)")
    B, N, H, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _expect(name, t, q8.shape, torch.uint8)
    if out is not None:
        _expect("out", out, q8.shape, torch.bfloat16)
    if lse is not None:
        _expect("lse", lse, (B, H, N), torch.float32)
    _check(q8, k8, v8, *(t for t in (out, lse) if t is not None))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, d), device=q8.device, dtype=torch.bfloat16)
    if lse is None:
        lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32)
    st = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                    scale, float(descale_q), float(descale_k), float(descale_v), int(causal), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return out, lse

