"""fa_bwd_atomic, the backward in one pass over the key tiles with dQ accumulated by fp32
atomics (head_dim 128, bf16), through the C ABI:

* against the oracle, element by element, at sizes that span several key tiles (128),
  query tiles (64) and ragged tails, padded and packed (with empty sequences), under the
  same tolerances as fa_bwd (gradients rel-L2 <= 3e-2);
* dK and dV against fa_bwd_preprocess + fa_bwd_dkdv on the same inputs, bitwise: the fused
  kernel runs the same dK/dV arithmetic in the same order, and the statistics come from
  the same kernel; its extra work (the masked first tile of the upper waves under causal
  masking, keys past the end) only adds exact zeros or is never stored;
* dQ against fa_bwd's deterministic dQ pass: both round dS to bf16 and sum in fp32, in
  different orders and with dS recomputed separately, so they differ by a few bf16 ulps
  of dS (rel-L2 well under 1e-2);
* run to run: dK and dV bitwise, dQ up to the order of the fp32 atomics (rel-L2 <= 1e-3);
* canary words around every output and the workspace;
* the full-size workloads bench.py times (B=4, H=32, N=4096 causal; 16384 packed tokens)
  on sampled heads / sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import check, f64

pytestmark = pytest.mark.gpu


def _w(causal: bool) -> W.Workload:
    return W.Workload("t_atomic", 1, 1, 1, 128, "bf16", causal, 1.0, 5151)


def _run(inp, causal, scale, deterministic):
    import exact_io_aware_attention_amd as fa
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    cu = inp.cu_seqlens.cuda() if inp.cu_seqlens is not None else None
    ms = inp.max_seqlen if cu is not None else None
    o, lse = fa.forward(q, k, v, causal=causal, softmax_scale=scale, cu_seqlens=cu, max_seqlen=ms)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, softmax_scale=scale, cu_seqlens=cu,
                             max_seqlen=ms, deterministic=deterministic)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _full_check(inp, causal, scale, label):
    o, lse, dq, dk, dv = _run(inp, causal, scale, False)
    cu = inp.cu_seqlens.numpy() if inp.cu_seqlens is not None else None
    o_r, lse_r = oracle.forward(inp.q, inp.k, inp.v, scale, causal, cu_seqlens=cu)
    dq_r, dk_r, dv_r = oracle.backward(inp.q, inp.k, inp.v, inp.do, scale, causal, cu_seqlens=cu)
    check(f"{label} O", "bf16", o, o_r, "o")
    check(f"{label} dQ", "bf16", dq, dq_r, "g")
    check(f"{label} dK", "bf16", dk, dk_r, "g")
    check(f"{label} dV", "bf16", dv, dv_r, "g")


SHAPES = [
    # (batch, seqlen, heads): one token, within one key tile, ragged tails on both tile
    # sizes, several key tiles, and 8 heads (the head-grouped workgroup order)
    (1, 1, 1), (2, 17, 3), (1, 64, 2), (1, 65, 2), (2, 128, 2), (1, 129, 2), (1, 200, 1),
    (1, 256, 2), (1, 300, 1), (1, 513, 1), (1, 384, 8),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_atomic_parity(causal, shape):
    B, N, H = shape
    w = _w(causal)
    inp = W.make_inputs(w, seed=6000 + 7 * N + H + causal, batch=B, seqlen=N, heads=H)
    _full_check(inp, causal, w.scale, f"atomic c{int(causal)} {B}x{N}x{H}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", [[1, 2, 127, 128, 129, 300, 64, 65], [0, 5, 0, 0, 130, 64, 0]],
                         ids=["ragged", "with_empty"])
def test_atomic_packed_parity(causal, lengths):
    w = _w(causal)
    inp = W.make_inputs(w, seed=6100 + len(lengths), heads=2, lengths=lengths)
    _full_check(inp, causal, w.scale, f"atomic packed c{int(causal)} {lengths}")


def _split_dkdv(inp, o, lse, causal, scale):
    """dK, dV from fa_bwd_preprocess then fa_bwd_dkdv (the statistics kernel the atomic
    path also runs)."""
    import exact_io_aware_attention_amd as fa
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    varlen = inp.cu_seqlens is not None
    cu = inp.cu_seqlens.cuda() if varlen else None
    B, N, H, d, T = inp.batch, inp.seqlen, q.shape[-2], q.shape[-1], inp.total_tokens
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, int(varlen), T)
    ws = torch.empty(max(wsb, 256), device="cuda", dtype=torch.uint8)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    sp = torch.cuda.current_stream().cuda_stream
    cup = cu.data_ptr() if varlen else None
    assert fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb, B, H, N, d, scale,
                                cup, T, fa.FA_DTYPE_BF16, sp) == fa.FA_OK
    assert fa.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                          wsb, dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, int(causal), cup, T,
                          fa.FA_DTYPE_BF16, sp) == fa.FA_OK
    torch.cuda.synchronize()
    return dk, dv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [(2, 333, 3, None), (1, 1000, 8, None), (0, 0, 2, [100, 0, 129, 128, 256])],
                         ids=["ragged", "8heads", "packed"])
def test_atomic_dkdv_bitwise_and_dq_close(causal, case):
    B, N, H, lengths = case
    w = _w(causal)
    if lengths is None:
        inp = W.make_inputs(w, seed=6200 + N, batch=B, seqlen=N, heads=H)
    else:
        inp = W.make_inputs(w, seed=6201, heads=H, lengths=lengths)
    o, lse, dq, dk, dv = _run(inp, causal, w.scale, False)
    dk_s, dv_s = _split_dkdv(inp, o, lse, causal, w.scale)
    assert torch.equal(dk, dk_s), "dK differs from fa_bwd_preprocess + fa_bwd_dkdv"
    assert torch.equal(dv, dv_s), "dV differs from fa_bwd_preprocess + fa_bwd_dkdv"
    dq_det = _run(inp, causal, w.scale, True)[2]
    a, b = f64(dq), f64(dq_det)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    print(f"dQ atomic vs deterministic: rel-L2 {rel:.3e}", flush=True)
    assert rel <= 1e-2


def test_atomic_runs_agree():
    w = _w(True)
    inp = W.make_inputs(w, seed=6300, batch=2, seqlen=700, heads=4)
    r1 = _run(inp, True, w.scale, False)
    r2 = _run(inp, True, w.scale, False)
    assert torch.equal(r1[3], r2[3]) and torch.equal(r1[4], r2[4])
    a, b = f64(r1[2]), f64(r2[2])
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    print(f"dQ run to run: rel-L2 {rel:.3e}", flush=True)
    assert rel <= 1e-3


def test_atomic_outputs_stay_in_bounds():
    """Canary words around every output buffer and around the workspace (whose
    accumulator takes the zero terms of the last query tile's rows past the end) stay
    untouched."""
    import exact_io_aware_attention_amd as fa
    w = _w(True)
    B, N, H, d = 1, 321, 3, 128
    inp = W.make_inputs(w, seed=6400, batch=B, seqlen=N, heads=H)
    pad = 4096
    n = B * N * H * d

    def guarded(numel, dtype, fill):
        buf = torch.full((numel + 2 * pad,), fill, device="cuda", dtype=dtype)
        return buf, buf[pad:pad + numel]

    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.forward(q, k, v, causal=True, softmax_scale=w.scale)
    grads = [guarded(n, torch.bfloat16, -1000.0) for _ in range(3)]
    dq, dk, dv = (x[1].view(B, N, H, d) for x in grads)
    wsb, ws = guarded(fa.fa_bwd_atomic_workspace_bytes(B, H, N, d, 0, 0), torch.uint8, 0xA5)
    fa.backward(q, k, v, o, lse, do, causal=True, softmax_scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                deterministic=False)
    torch.cuda.synchronize()
    for buf, fill in [(wsb, 0xA5)] + [(x[0], -1000.0) for x in grads]:
        edges = torch.cat([buf[:pad], buf[-pad:]]).float().cpu().numpy()
        assert np.all(edges == fill)
    dq_r, dk_r, dv_r = oracle.backward(inp.q, inp.k, inp.v, inp.do, w.scale, True)
    check("canary case dQ", "bf16", dq, dq_r, "g")


def test_atomic_c3_full_size_sampled_heads():
    w = W.get("c3")
    inp = W.make_inputs(w)
    o, lse, dq, dk, dv = _run(inp, w.causal, w.scale, False)
    for b, h in [(0, 3), (3, 30)]:
        q, k, v, do = (oracle.to_f64(x[b, :, h, :]) for x in (inp.q, inp.k, inp.v, inp.do))
        dq_r, dk_r, dv_r = oracle.head_backward(q, k, v, do, w.scale, w.causal)
        tag = f"atomic c3 b{b} h{h}"
        check(f"{tag} dQ", "bf16", dq[b, :, h, :], dq_r, "g")
        check(f"{tag} dK", "bf16", dk[b, :, h, :], dk_r, "g")
        check(f"{tag} dV", "bf16", dv[b, :, h, :], dv_r, "g")


def test_atomic_c5_full_size_sampled_sequences():
    w = W.get("c5")
    inp = W.make_inputs(w)
    o, lse, dq, dk, dv = _run(inp, True, w.scale, False)
    cu = inp.cu_seqlens.tolist()
    nseq = len(cu) - 1
    for s, h in [(1, 5), (nseq - 1, 31)]:
        a, e = cu[s], cu[s + 1]
        q, k, v, do = (oracle.to_f64(x[a:e, h, :]) for x in (inp.q, inp.k, inp.v, inp.do))
        dq_r, dk_r, dv_r = oracle.head_backward(q, k, v, do, w.scale, True)
        tag = f"atomic c5 seq{s} (len {e - a}) h{h}"
        check(f"{tag} dQ", "bf16", dq[a:e, h, :], dq_r, "g")
        check(f"{tag} dK", "bf16", dk[a:e, h, :], dk_r, "g")
        check(f"{tag} dV", "bf16", dv[a:e, h, :], dv_r, "g")
