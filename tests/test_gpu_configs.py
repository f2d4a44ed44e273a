"""The five workloads at full size, in the launch configuration the benchmark times,
checked against the oracle on outputs it can compute one by one:

* c1 (1x1x128, d=64, fp32): every output.
* c2 (8x16x2048, d=64) and c3 (4x32x4096, d=128, causal): whole heads sampled from
  the batch (each head is independent of the others).
* c4 (1x8x65536, d=64): O, LSE and dQ on 256 seeded query rows of every head, and dK
  and dV on 256 seeded key rows of every head. A key row's gradients sum over every
  query row's softmax, which costs the oracle about a minute per head, so those
  expected values were computed once by tests/golden/make_c4_key_rows.py (the oracle
  alone, on the same seeded inputs, whose digests the file records) and are read from
  tests/golden/c4_key_rows.npz. Gradient identities that hold at any size cover every
  row, and exact parity of whole heads runs at the same settings with N = 8192. Memory:
  the library allocates nothing and its workspace is O(N).
* c5 (16384 packed tokens, causal per sequence): sampled sequences x heads, including
  the truncated last sequence.
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import check, f64, run_gpu

pytestmark = pytest.mark.gpu

GOLDEN_C4 = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c4_key_rows.npz")


def _head(t, b, h):
    return oracle.to_f64(t[b, :, h, :])


def _check_heads(inp, w, outs, heads, label):
    o, lse, dq, dk, dv = outs
    for b, h in heads:
        q, k, v, do = (_head(x, b, h) for x in (inp.q, inp.k, inp.v, inp.do))
        o_r, l_r = oracle.head_forward(q, k, v, w.scale, w.causal)
        dq_r, dk_r, dv_r = oracle.head_backward(q, k, v, do, w.scale, w.causal)
        tag = f"{label} b{b} h{h}"
        check(f"{tag} O", w.dtype, o[b, :, h, :], o_r, "o")
        check(f"{tag} LSE", w.dtype, lse[b, h, :], l_r, "lse")
        check(f"{tag} dQ", w.dtype, dq[b, :, h, :], dq_r, "g")
        check(f"{tag} dK", w.dtype, dk[b, :, h, :], dk_r, "g")
        check(f"{tag} dV", w.dtype, dv[b, :, h, :], dv_r, "g")


def test_c1_full():
    w = W.get("c1")
    inp = W.make_inputs(w)
    _check_heads(inp, w, run_gpu(inp, w.causal, w.scale), [(0, 0)], "c1")


def test_c2_sampled_heads():
    w = W.get("c2")
    inp = W.make_inputs(w)
    _check_heads(inp, w, run_gpu(inp, w.causal, w.scale), [(0, 0), (3, 7), (7, 15)], "c2")


def test_c3_sampled_heads():
    w = W.get("c3")
    inp = W.make_inputs(w)
    _check_heads(inp, w, run_gpu(inp, w.causal, w.scale), [(0, 0), (1, 17), (3, 31)], "c3")


def test_c5_sampled_sequences():
    w = W.get("c5")
    inp = W.make_inputs(w)
    o, lse, dq, dk, dv = run_gpu(inp, w.causal, w.scale)
    cu = inp.cu_seqlens.tolist()
    nseq = len(cu) - 1
    for s, h in [(0, 0), (nseq // 2, 13), (nseq - 1, 31)]:
        a, e = cu[s], cu[s + 1]
        q, k, v, do = (oracle.to_f64(x[a:e, h, :]) for x in (inp.q, inp.k, inp.v, inp.do))
        o_r, l_r = oracle.head_forward(q, k, v, w.scale, True)
        dq_r, dk_r, dv_r = oracle.head_backward(q, k, v, do, w.scale, True)
        tag = f"c5 seq{s} (len {e - a}) h{h}"
        check(f"{tag} O", "bf16", o[a:e, h, :], o_r, "o")
        check(f"{tag} LSE", "bf16", lse[h, a:e], l_r, "lse")
        check(f"{tag} dQ", "bf16", dq[a:e, h, :], dq_r, "g")
        check(f"{tag} dK", "bf16", dk[a:e, h, :], dk_r, "g")
        check(f"{tag} dV", "bf16", dv[a:e, h, :], dv_r, "g")


def test_c4_full_size():
    import exact_io_aware_attention_amd as fa
    w = W.get("c4")
    inp = W.make_inputs(w)
    outs = run_gpu(inp, w.causal, w.scale)
    o, lse, dq, dk, dv = outs
    rows = W.sample_rows(w.seed, w.seqlen, 256)
    for h in range(w.heads):
        q, k, v, do = (_head(x, 0, h) for x in (inp.q, inp.k, inp.v, inp.do))
        o_r, l_r = oracle.forward_rows(q, k, v, w.scale, False, rows)
        dq_r = oracle.backward_query_rows(q, k, v, do, w.scale, False, rows)
        check(f"c4 h{h} O[256 rows]", "bf16", o[0, rows, h, :], o_r, "o")
        check(f"c4 h{h} LSE[256 rows]", "bf16", lse[0, h, rows], l_r, "lse")
        check(f"c4 h{h} dQ[256 rows]", "bf16", dq[0, rows, h, :], dq_r, "g")
        # Gradient identities (any size): rows of P sum to one, so sum_j dV_j = sum_i dO_i;
        # rows of dS sum to zero, so sum_j dK_j = 0; and tr(Q^T dQ) = tr(K^T dK). The
        # gradient contract allows a per-tensor relative error (rel-L2) of 3e-2, i.e. an
        # rms error of 3e-2 * rms(g) per element; summed with random signs over N rows
        # that gives a standard deviation of sqrt(N) * 3e-2 * rms(g) per column, and the
        # bound is three of those.
        dvh, dkh, dqh = f64(dv[0, :, h, :]), f64(dk[0, :, h, :]), f64(dq[0, :, h, :])
        n = dvh.shape[0]
        want = do.sum(axis=0)
        err_v = np.abs(dvh.sum(axis=0) - want).max()
        assert err_v <= 3 * 3e-2 * np.sqrt(n) * np.sqrt((dvh ** 2).mean()), (h, err_v)
        err_k = np.abs(dkh.sum(axis=0)).max()
        assert err_k <= 3 * 3e-2 * np.sqrt(n) * np.sqrt((dkh ** 2).mean()), (h, err_k)
        tq, tk = np.sum(q * dqh), np.sum(k * dkh)
        assert abs(tq - tk) <= 3e-2 * max(abs(tq), np.sqrt(n) * np.sqrt((dqh ** 2).mean())), (h, tq, tk)
        print(f"c4 h{h} identities: |sum dV - sum dO| {err_v:.3e} |sum dK| {err_k:.3e} "
              f"tr(Q'dQ) {tq:.4e} tr(K'dK) {tk:.4e}", flush=True)
    # dK and dV, element by element, on 256 seeded key rows of every head.
    gold = np.load(GOLDEN_C4)
    digests = [hashlib.sha256(t.contiguous().view(-1).view(torch.uint8).numpy().tobytes()).hexdigest()
               for t in (inp.q, inp.k, inp.v, inp.do)]
    assert list(gold["sha256"]) == digests, "c4 inputs differ from those the stored key rows were computed on"
    keys = gold["keys"]
    assert np.array_equal(keys, W.sample_rows(w.seed + 100, w.seqlen, 256))
    for h in range(w.heads):
        check(f"c4 h{h} dK[256 key rows]", "bf16", dk[0, keys, h, :], gold["dk"][h].astype(np.float64), "g")
        check(f"c4 h{h} dV[256 key rows]", "bf16", dv[0, keys, h, :], gold["dv"][h].astype(np.float64), "g")


def test_c4_library_allocates_nothing():
    """Linear memory: with every buffer allocated by the caller up front, the forward
    and backward calls leave the device's free memory unchanged, and the only scratch
    they need (the workspace) is two fp32 per (head, row) and 256 bytes of work
    counters: O(N), where one head's N x N fp32 score matrix alone would be 17 GB."""
    import exact_io_aware_attention_amd as fa
    w = W.get("c4")
    B, N, H, d = 1, w.seqlen, w.heads, w.head_dim
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    q, k, v, do = (torch.randn(B, N, H, d, device=dev, generator=g).to(torch.bfloat16) for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(B, H, N, device=dev, dtype=torch.float32)
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d, 0, 0)
    assert ws_bytes == 2 * H * N * 4 + 256 and ws_bytes < 1e-3 * N * N * 4
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    sp = torch.cuda.current_stream().cuda_stream
    assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                     w.scale, 0, None, 0, fa.FA_DTYPE_BF16, sp) == fa.FA_OK
    assert fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N, d,
                     w.scale, 0, None, 0, fa.FA_DTYPE_BF16, sp) == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()


def test_c4_settings_exact_dk_dv_at_n8192():
    w = W.get("c4")
    inp = W.make_inputs(w, seqlen=8192)
    _check_heads(inp, w, run_gpu(inp, w.causal, w.scale), [(0, 0), (0, 5)], "c4@8192")
