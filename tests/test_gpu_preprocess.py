"""The backward's row statistics through the C ABI: the workspace that fa_bwd_preprocess,
and the dQ pass that forms them itself (fa_bwd_dq_stats, what fa_bwd runs), write
(D_i = sum_k dO_ik O_ik of the stored O, then -LSE_i / scale, each an fp32 array in the
LSE layout starting on a 256-byte boundary) against the oracle's backward statistics,
element by element; and the work counters behind them (256 bytes the dK/dV stage hands
its key tiles out with): zero after either producer, zero again after every dK/dV call,
so that dK/dV called twice on one workspace gives the same bits.

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


@pytest.mark.parametrize("producer", ["preprocess", "dq_stats"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_preprocess_matches_oracle(case, producer):
    label, dtype, B, N, H, d, cu = case
    print(f"statistics from {producer}: {label}", flush=True)
    g = torch.Generator().manual_seed(77 + N + H)
    T = cu[-1] if cu is not None else B * N
    shape = (T, H, d) if cu is not None else (B, N, H, d)
    o = torch.randn(shape, generator=g).to(dtype)
    do = torch.randn(shape, generator=g).to(dtype)
    lse_shape = (H, T) if cu is not None else (B, H, N)
    lse = (torch.randn(lse_shape, generator=g) * 4.0).float()
    scale = 0.0883883
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d, int(cu is not None), T)
    assert ws_bytes == 2 * _stat_bytes(H, T) + 256
    ws = torch.full((ws_bytes,), 0xA5, device="cuda", dtype=torch.uint8)
    od, dod, lsed = o.cuda(), do.cuda(), lse.cuda()
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    code = fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_FP32
    cup = cud.data_ptr() if cud is not None else None
    sp = torch.cuda.current_stream().cuda_stream
    if producer == "preprocess":
        st = fa.fa_bwd_preprocess(od.data_ptr(), dod.data_ptr(), lsed.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N,
                                  d, scale, cup, T, code, sp)
    else:
        # the dQ pass needs Q, K, V too; only the statistics it leaves are checked here
        q, k, v = (torch.randn(shape, generator=g).to(dtype).cuda() for _ in range(3))
        dq = torch.empty_like(q)
        st = fa.fa_bwd_dq_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), dod.data_ptr(),
                                lsed.data_ptr(), ws.data_ptr(), ws_bytes, dq.data_ptr(), B, H, N, d, scale, 1, cup,
                                T, code, sp)
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
    # the nine work counters of the dK/dV stage start at zero (the rest of the block is unused)
    ctr = raw[2 * off: 2 * off + 36].view(torch.int32)
    assert torch.all(ctr == 0), f"{label}: counters {ctr.tolist()}"


DKDV_CASES = [
    # (label, batch, seqlen, heads, cu_seqlens, causal)
    ("d128 causal ragged", 2, 333, 3, None, 1),
    ("d128 non-causal", 1, 700, 4, None, 0),
    ("d128 packed", 3, 257, 2, [0, 100, 101, 358], 1),
    ("d128 packed with empty key tiles", 4, 600, 2, [0, 600, 610, 1000, 1130], 1),
]


@pytest.mark.parametrize("case", DKDV_CASES, ids=[c[0] for c in DKDV_CASES])
def test_dkdv_twice_on_one_workspace(case):
    label, B, N, H, cu, causal = case
    print(f"dK/dV twice: {label}", flush=True)
    d = 128
    g = torch.Generator().manual_seed(5 + N + H)
    T = cu[-1] if cu is not None else B * N
    shape = (T, H, d) if cu is not None else (B, N, H, d)
    q, k, v, do = (torch.randn(shape, generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    cup = cud.data_ptr() if cud is not None else None
    lse_shape = (H, T) if cu is not None else (B, H, N)
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, device="cuda", dtype=torch.float32)
    scale = d ** -0.5
    bf = fa.FA_DTYPE_BF16
    sp = torch.cuda.current_stream().cuda_stream
    assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, scale,
                     causal, cup, T, bf, sp) == fa.FA_OK
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d, int(cu is not None), T)
    ws = torch.full((ws_bytes,), 0xA5, device="cuda", dtype=torch.uint8)
    dq = torch.empty_like(q)
    assert fa.fa_bwd_dq_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              ws.data_ptr(), ws_bytes, dq.data_ptr(), B, H, N, d, scale, causal, cup, T, bf,
                              sp) == fa.FA_OK
    off = 2 * _stat_bytes(H, T)
    runs = []
    for _ in range(2):
        dk, dv = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
        assert fa.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                              ws_bytes, dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, causal, cup, T, bf,
                              sp) == fa.FA_OK
        torch.cuda.synchronize()
        ctr = ws[off: off + 36].cpu().view(torch.int32)
        assert torch.all(ctr == 0), f"{label}: counters left at {ctr.tolist()}"
        assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all(), f"{label}: rows left unwritten"
        runs.append((dk.cpu(), dv.cpu()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1]), label
