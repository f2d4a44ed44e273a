"""The C ABI on the CPU: the library loads, exports what include/fa.h declares, and
rejects bad arguments with the documented codes before any HIP call (no GPU here)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_io_aware_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

A = 1 << 20          # a 16-byte-aligned fake device address: never dereferenced on these paths
MIS = A + 2          # misaligned


def _lib():
    if not os.path.exists(fa.library_path()):
        pytest.skip("libfa.so not built (python -m exact_io_aware_attention_amd.build)")
    return fa.load_library()


def declared_functions(headers=(HEADER,)):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_bwd", "fa_bwd_atomic", "fa_bwd_atomic_workspace_bytes", "fa_bwd_dkdv",
                                    "fa_bwd_dq", "fa_bwd_dq_stats", "fa_bwd_noalloc", "fa_bwd_preprocess",
                                    "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_decode",
                                    "fa_fwd_decode_workspace_bytes", "fa_fwd_fp8", "fa_strerror"]


def test_measurement_header_declares_its_calls():
    assert declared_functions([os.path.join(ROOT, "include", "fa_ubench.h")]) == [
        "fa_device_info", "fa_ubench_copy", "fa_ubench_lds", "fa_ubench_mfma_bf16", "fa_ubench_mfma_fp8", "fa_ubench_mfma_mix", "fa_ubench_mfma_valu",
        "fa_ubench_valu"]


def test_library_exports_every_declared_symbol():
    lib = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert len(HEADERS) >= 2
    for name in declared_functions(HEADERS):
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_has_no_undefined_internal_symbols():
    """Every kernel launch stub is defined (a host-pass miscompile once left them
    undefined, which only shows up as a load failure on a machine with a GPU)."""
    _lib()
    out = subprocess.run(["nm", "-D", fa.library_path()], capture_output=True, text=True, check=True).stdout
    missing = [l for l in out.splitlines() if " U " in l and "_ZN2fa" in l]
    assert missing == []


def _fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, heads=1, seqlen=16, head_dim=64, softmax_scale=0.125,
                causal=0, cu_seqlens=None, total_tokens=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


def _bwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, workspace=A, workspace_bytes=1 << 30,
                batch=1, heads=1, seqlen=16, head_dim=64, softmax_scale=0.125, causal=0, cu_seqlens=None,
                total_tokens=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(batch=0), fa.FA_ERR_INVALID_ARG),
    (dict(heads=-1), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),    # the scale must be positive
    (dict(softmax_scale=-0.125), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.0), fa.FA_ERR_INVALID_ARG),
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(cu_seqlens=A, total_tokens=-1), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens=A + 1, total_tokens=4), fa.FA_ERR_INVALID_ARG),
    (dict(batch=1 << 20, heads=1 << 12, seqlen=1 << 12), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens=A, total_tokens=0), fa.FA_OK),   # empty packed batch: nothing to launch
])
def test_fwd_argument_checks(kw, code):
    _lib()
    assert _fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(head_dim=32), fa.FA_ERR_UNSUPPORTED),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),   # the scale must be positive
    (dict(softmax_scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(workspace_bytes=255), fa.FA_ERR_WORKSPACE),
    (dict(workspace=A + 16), fa.FA_ERR_WORKSPACE),
    (dict(seqlen=-5), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens=A, total_tokens=0), fa.FA_OK),
])
def test_bwd_argument_checks(kw, code):
    _lib()
    assert _bwd(**kw) == code


def test_stage_argument_checks():
    _lib()
    common = dict(batch=1, heads=2, seqlen=16, head_dim=64, cu_seqlens=None, total_tokens=0,
                  dtype=fa.FA_DTYPE_BF16, stream=None)
    ws = dict(workspace=A, workspace_bytes=1 << 20)
    pre = dict(softmax_scale=0.125)
    assert fa.fa_bwd_preprocess(o=None, dout=A, lse=A, **ws, **pre, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=None, **ws, **pre, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=MIS, **ws, **pre, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=A, workspace=None, workspace_bytes=0, **pre,
                                **common) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=A, **ws, softmax_scale=0.0, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=A, **ws, softmax_scale=-0.5, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dkdv(q=A, k=A, v=A, dout=A, lse=A, dk=A, dv=A, **ws, softmax_scale=-0.1, causal=0,
                          **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq(q=A, k=A, v=A, dout=A, lse=A, dq=A, **ws, softmax_scale=0.0, causal=0,
                        **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_preprocess(o=A, dout=A, lse=A, **ws, **pre, **dict(common, head_dim=48)) == fa.FA_ERR_UNSUPPORTED
    sc = dict(softmax_scale=0.125, causal=1)
    assert fa.fa_bwd_dkdv(q=A, k=A, v=A, dout=A, lse=A, dk=None, dv=A, **ws, **sc, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dkdv(q=A, k=A, v=A, dout=A, lse=A, dk=A, dv=A, workspace=A, workspace_bytes=64,
                          **sc, **common) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dq(q=A, k=A, v=MIS, dout=A, lse=A, dq=A, **ws, **sc, **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq(q=A, k=A, v=A, dout=A, lse=A, dq=A, **ws, **dict(sc, causal=-1),
                        **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq_stats(q=A, k=A, v=A, o=None, dout=A, lse=A, dq=A, **ws, **sc,
                              **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq_stats(q=A, k=A, v=A, o=MIS, dout=A, lse=A, dq=A, **ws, **sc,
                              **common) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq_stats(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, workspace=A, workspace_bytes=8,
                              **sc, **common) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dq_stats(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, **ws, softmax_scale=-1.0, causal=0,
                              **common) == fa.FA_ERR_INVALID_ARG


def _atomic(**kw):
    args = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, workspace=A, workspace_bytes=1 << 30,
                batch=1, heads=2, seqlen=16, head_dim=128, softmax_scale=0.125, causal=1, cu_seqlens=None,
                total_tokens=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_bwd_atomic(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(head_dim=64), fa.FA_ERR_UNSUPPORTED),          # the fused kernel is built for 128
    (dict(dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=32), fa.FA_ERR_UNSUPPORTED),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace=A + 16), fa.FA_ERR_WORKSPACE),
    # room for fa_bwd's statistics and work counters but not for the accumulator
    (dict(workspace_bytes=3 * 256), fa.FA_ERR_WORKSPACE),
    (dict(cu_seqlens=A, total_tokens=0), fa.FA_OK),
])
def test_atomic_bwd_argument_checks(kw, code):
    _lib()
    assert _atomic(**kw) == code


def test_atomic_workspace_size():
    _lib()
    # fa_bwd's statistics, then (heads * tokens + 64) rows of head_dim fp32
    assert fa.fa_bwd_atomic_workspace_bytes(4, 32, 4096, 128, 0, 0) == (
        2 * 4 * 32 * 4096 * 4 + 256 + (32 * 4 * 4096 + 64) * 128 * 4)
    assert fa.fa_bwd_atomic_workspace_bytes(1, 2, 16, 128, 0, 0) == 2 * 256 + 256 + (2 * 16 + 64) * 128 * 4
    assert fa.fa_bwd_atomic_workspace_bytes(7, 32, 2048, 128, 1, 16384) == (
        2 * 32 * 16384 * 4 + 256 + (32 * 16384 + 64) * 128 * 4)
    assert fa.fa_bwd_atomic_workspace_bytes(1, 1, 1, 80, 0, 0) == 0
    assert _atomic(workspace_bytes=fa.fa_bwd_atomic_workspace_bytes(1, 2, 16, 128, 0, 0) - 4) == fa.FA_ERR_WORKSPACE


def test_workspace_size():
    _lib()
    # two fp32 arrays (D and -LSE / scale), each rounded up to 256 bytes
    # two statistics arrays (each rounded up to 256 bytes), then 256 bytes of work counters
    assert fa.fa_bwd_workspace_bytes(4, 32, 4096, 128, 0, 0) == 2 * 4 * 32 * 4096 * 4 + 256
    assert fa.fa_bwd_workspace_bytes(1, 3, 5, 64, 0, 0) == 2 * 256 + 256
    assert fa.fa_bwd_workspace_bytes(7, 32, 2048, 128, 1, 16384) == 2 * 32 * 16384 * 4 + 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 80, 0, 0) == 0
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64, 0, 0) == 0


def test_strerror_covers_every_code():
    _lib()
    seen = set()
    for code in range(6):
        s = fa.fa_strerror(code)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in fa.fa_strerror(99)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "library_path", lambda: str(tmp_path / "libfa.so"))
    with pytest.raises(RuntimeError, match="not found"):
        fa.load_library()


# ---------------------------------------------------------------- decode

def _dec(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, heads=2, seqlen_q=4, seqlen_k=1000, head_dim=128,
                softmax_scale=0.1, causal=1, num_splits=0, workspace=None, workspace_bytes=0,
                dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd_decode(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_k=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_q=33), fa.FA_ERR_UNSUPPORTED),
    (dict(seqlen_q=8, seqlen_k=4, causal=1), fa.FA_ERR_INVALID_ARG),
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=17), fa.FA_ERR_INVALID_ARG),  # more splits than 64-key chunks
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(softmax_scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(), fa.FA_ERR_WORKSPACE),                                   # no workspace
    (dict(workspace=A, workspace_bytes=16), fa.FA_ERR_WORKSPACE),    # too small
    (dict(workspace=A + 16, workspace_bytes=1 << 30), fa.FA_ERR_WORKSPACE),  # not 256-aligned
])
def test_decode_rejects_bad_arguments(kw, code):
    _lib()
    assert _dec(**kw) == code


def test_decode_workspace_size():
    _lib()
    # 1024 / (B*H) splits, each at least 256 keys: B*H = 256 -> 4 splits of 4096 keys
    assert fa.fa_fwd_decode_workspace_bytes(8, 32, 1, 16384, 128, 0) == 256 * 4 * 1 * (128 + 1) * 4 // 256 * 256 + \
        (256 if (256 * 4 * 129 * 4) % 256 else 0)
    # explicit split count: 4 splits of 64 keys (256 keys), 5 queries, d = 64
    want = 2 * 3 * 4 * 5 * (64 + 1) * 4
    assert fa.fa_fwd_decode_workspace_bytes(2, 3, 5, 256, 64, 4) == (want + 255) // 256 * 256
    # splits are whole multiples of 64 keys: 3 requested over 200 keys gives 2 of 128
    want = 2 * 3 * 2 * 5 * (64 + 1) * 4
    assert fa.fa_fwd_decode_workspace_bytes(2, 3, 5, 200, 64, 3) == (want + 255) // 256 * 256
    assert fa.fa_fwd_decode_workspace_bytes(1, 1, 33, 100, 128, 0) == 0   # unsupported
    assert fa.fa_fwd_decode_workspace_bytes(1, 1, 1, 100, 128, 3) == 0    # > ceil(100 / 64) splits


# ---------------------------------------------------------------- 8-bit forward

def _fp8(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, heads=2, seqlen=100, head_dim=128, softmax_scale=0.1,
                descale_q=1.0, descale_k=1.0, descale_v=1.0, causal=1, stream=None)
    args.update(kw)
    return fa.fa_fwd_fp8(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(o=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen=0), fa.FA_ERR_INVALID_ARG),
    (dict(batch=-1), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(descale_q=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(descale_v=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(descale_q=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_k=-2.0), fa.FA_ERR_INVALID_ARG),
    (dict(descale_q=1e-30, descale_k=1e-30), fa.FA_ERR_INVALID_ARG),  # the product underflows to 0
    (dict(head_dim=96), fa.FA_ERR_UNSUPPORTED),
])
def test_fp8_argument_checks(kw, code):
    _lib()
    assert _fp8(**kw) == code



# ---------------------------------------------------------------- measurement calls

def test_ubench_argument_checks():
    _lib()
    assert fa.fa_ubench_mfma_bf16(None, 1, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_bf16(A, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_fp8(None, 1, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_fp8(A, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_fp8(A, 1, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_valu(A, 1, 0, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_valu(A, 1, 1, 2, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_lds(A, 1, 1, 5, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_lds(None, 1, 1, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_copy(A, A + 4096, 100, 8, None) == fa.FA_ERR_INVALID_ARG   # not a multiple of 16
    assert fa.fa_ubench_mfma_valu(A, 1, 1, 3, 0, 0, None) == fa.FA_ERR_INVALID_ARG  # nvalu not 0, 2, 4, 8
    assert fa.fa_ubench_mfma_valu(A, 1, 1, 4, 2, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_valu(A, 1, 1, 4, 0, 2, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_valu(None, 1, 1, 4, 0, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_valu(A, 0, 1, 4, 0, 0, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_mix(A, 1, 1, 2, None) == fa.FA_ERR_INVALID_ARG  # mix not 0 or 1
    assert fa.fa_ubench_mfma_mix(None, 1, 1, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_mix(A, 0, 1, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_mfma_mix(A, 1, 0, 1, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_copy(A + 8, A + 4096, 256, 8, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_ubench_copy(A, A + 4096, 256, 0, None) == fa.FA_ERR_INVALID_ARG


# ---------------------------------------------------------------- backward without allocation

def _noalloc(**kw):
    args = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, batch=1, heads=1, seqlen=16, head_dim=64,
                softmax_scale=0.125, causal=0, cu_seqlens=None, total_tokens=0, dtype=fa.FA_DTYPE_BF16,
                stream=None)
    args.update(kw)
    return fa.fa_bwd_noalloc(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(dq=None), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(head_dim=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dv=MIS), fa.FA_ERR_INVALID_ARG),
    # 8 bytes per (head, token): 2^21 pairs fit the 16 MiB array, one token more does not
    (dict(batch=1, heads=32, seqlen=65537), fa.FA_ERR_SCRATCH),
    (dict(batch=2, heads=16, seqlen=65536 + 64), fa.FA_ERR_SCRATCH),
    (dict(cu_seqlens=A, total_tokens=(1 << 21) + 1, seqlen=2048, batch=4), fa.FA_ERR_SCRATCH),
    (dict(cu_seqlens=A, total_tokens=0), fa.FA_OK),   # empty packed batch: nothing to launch
])
def test_noalloc_argument_checks(kw, code):
    _lib()
    assert _noalloc(**kw) == code
    assert fa.FA_BWD_NOALLOC_MAX_SCRATCH == (16 << 20) + 256
