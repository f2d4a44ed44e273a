"""fa_bwd_preprocess through the C ABI: the workspace it writes (D_i = sum_k dO_ik O_ik
of the stored O, then -LSE_i / scale, each an fp32 array in the LSE layout starting on a
256-byte boundary) against the oracle's backward statistics, element by element.

Bound for D: the kernel forms exact products of bf16 values and adds them in fp32, so
|D - D_ref| <= n u sum_k |dO_ik O_ik| with n = head_dim terms and u = 2^-24; 1e-5 covers
n = 128 (7.6e-6). fp32 inputs add one rounding per product: (n + 1) u, still below 1e-5.
-LSE / scale is one fp32 division: relative 2^-24.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_attention_amd as fa
import oracle

pytestmark = pytest.mark.gpu

CASES = [
    # (label, dtype, batch, seqlen, heads, head_dim, cu_seqlens)
    ("bf16 d128 ragged", torch.bfloat16, 2, 333, 3, 128, None),
    ("bf16 d64 one tile", torch.bfloat16, 1, 64, 2, 64, None),
    ("bf16 d128 single token", torch.bfloat16, 3, 1, 2, 128, None),
    ("bf16 d128 packed", torch.bfloat16, 3, 257, 2, 128, [0, 100, 101, 358]),
    ("bf16 d64 packed", torch.bfloat16, 2, 200, 5, 64, [0, 200, 263]),
    ("fp32 d64 ragged", torch.float32, 1, 70, 2, 64, None),
    ("bf16 d128 llama-shaped", torch.bfloat16, 1, 4096, 32, 128, None),
]


def _stat_bytes(heads, tokens):
    return (heads * tokens * 4 + 255) // 256 * 256


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_preprocess_matches_oracle(case):
    label, dtype, B, N, H, d, cu = case
    print(f"preprocess {label}", flush=True)
    g = torch.Generator().manual_seed(77 + N + H)
    T = cu[-1] if cu is not None else B * N
    shape = (T, H, d) if cu is not None else (B, N, H, d)
    o = torch.randn(shape, generator=g).to(dtype)
    do = torch.randn(shape, generator=g).to(dtype)
    lse_shape = (H, T) if cu is not None else (B, H, N)
    lse = (torch.randn(lse_shape, generator=g) * 4.0).float()
    scale = 0.0883883
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d, int(cu is not None), T)
    assert ws_bytes == 2 * _stat_bytes(H, T)
    ws = torch.full((ws_bytes,), 0xA5, device="cuda", dtype=torch.uint8)
    od, dod, lsed = o.cuda(), do.cuda(), lse.cuda()
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    code = fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_FP32
    st = fa.fa_bwd_preprocess(od.data_ptr(), dod.data_ptr(), lsed.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d,
                              scale, cud.data_ptr() if cud is not None else None, T, code,
                              torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    raw = ws.cpu()
    n = H * T
    dvec = raw[: 4 * n].view(torch.float32).numpy().astype(np.float64).reshape(lse_shape)
    off = _stat_bytes(H, T)
    mneg = raw[off: off + 4 * n].view(torch.float32).numpy().astype(np.float64).reshape(lse_shape)
    d_ref, m_ref = oracle.backward_stats(o, do, lse, scale, cu_seqlens=np.array(cu) if cu is not None else None)
    mag = np.abs(oracle.to_f64(o) * oracle.to_f64(do)).sum(axis=-1)
    mag = mag.transpose(0, 2, 1) if cu is None else mag.T
    err_d = np.abs(dvec - d_ref)
    assert np.all(err_d <= 1e-5 * mag + 1e-30), f"{label}: D off by {err_d.max()} (worst ratio {(err_d / (mag + 1e-30)).max()})"
    np.testing.assert_allclose(mneg, m_ref, rtol=2.0 ** -23, atol=0)
