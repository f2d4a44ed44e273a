"""HIP path vs the CPU oracle, element by element, on seeded inputs small enough for
the oracle to finish in seconds while still spanning several tiles and ragged tails
(query tiles of 128, key tiles of 64, backward key tiles of 128 and query tiles of 64).
"""
import numpy as np
import pytest
import torch

import workloads as W
import oracle
from parity_utils import check, f64, full_parity, run_gpu

pytestmark = pytest.mark.gpu


def _w(dtype: str, d: int, causal: bool, std: float = 1.0) -> W.Workload:
    return W.Workload(f"t_{dtype}_{d}", 1, 1, 1, d, dtype, causal, std, 4242)


SHAPES = [
    # (batch, seqlen, heads)
    (1, 1, 1), (2, 17, 3), (1, 64, 2), (1, 65, 2), (1, 127, 1), (2, 128, 2), (1, 129, 2),
    (1, 200, 1), (1, 256, 2), (1, 300, 1), (1, 513, 1),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_parity(d, causal, shape):
    B, N, H = shape
    w = _w("bf16", d, causal)
    inp = W.make_inputs(w, seed=1000 + N * 7 + d + causal, batch=B, seqlen=N, heads=H)
    full_parity(inp, causal, w.scale, "bf16", f"bf16 d{d} c{int(causal)} {B}x{N}x{H}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 77, 2), (1, 128, 1), (2, 200, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp32_parity(d, causal, shape):
    B, N, H = shape
    w = _w("fp32", d, causal)
    inp = W.make_inputs(w, seed=2000 + N + d, batch=B, seqlen=N, heads=H)
    full_parity(inp, causal, w.scale, "fp32", f"fp32 d{d} c{int(causal)} {B}x{N}x{H}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_parity(dtype, d, causal):
    lengths = [1, 2, 127, 128, 129, 300, 64, 65]
    w = _w(dtype, d, causal)
    inp = W.make_inputs(w, seed=3000 + d, heads=2, lengths=lengths)
    full_parity(inp, causal, w.scale, dtype, f"packed {dtype} d{d} c{int(causal)}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_with_empty_sequences(dtype, d, causal):
    """Zero-length sequences in a packed batch (first, between others, last) own no
    tokens: every kernel skips them and the other sequences are unaffected."""
    lengths = [0, 5, 0, 0, 130, 64, 0]
    w = _w(dtype, d, causal)
    inp = W.make_inputs(w, seed=3100 + d, heads=2, lengths=lengths)
    assert inp.cu_seqlens.tolist() == [0, 0, 5, 5, 5, 135, 199, 199]
    full_parity(inp, causal, w.scale, dtype, f"packed with empty {dtype} d{d} c{int(causal)}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_peaky_softmax(d, causal):
    """Q and K scaled by 8 (exact in bf16): near one-hot rows stress the running max and
    its rescale; V and dO keep unit scale so the absolute bounds keep their meaning."""
    w = _w("bf16", d, causal)
    inp = W.make_inputs(w, seed=77, batch=1, seqlen=257, heads=2)
    inp.q.mul_(8)
    inp.k.mul_(8)
    full_parity(inp, causal, w.scale, "bf16", f"peaky d{d} c{int(causal)}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_growing_along_keys(d, causal):
    """Every query gets a common component u (a +-1 pattern per head) and the keys drift
    along u with their position, so the scores of each later key block exceed the running
    reference by far more than 2^8: the forward moves its reference (its uncommon path)
    on most blocks instead of on a query tile's first one only. Only O and LSE are held to
    the contract: the reference moves are the forward's, and with rows this close to
    one-hot each dS = P (dP - D) is a difference of nearly equal terms (D comes from the
    bf16 O), so the gradients' relative error says nothing here (as with identical keys)."""
    w = _w("bf16", d, causal)
    inp = W.make_inputs(w, seed=91, batch=1, seqlen=600, heads=2)
    n = inp.k.shape[1]
    u = torch.sign(inp.q[:, :1].float())
    inp.q.copy_((inp.q.float() + 0.5 * u).to(inp.q.dtype))
    drift = 0.05 * torch.arange(n, dtype=torch.float32)[None, :, None, None] * u
    inp.k.copy_((inp.k.float() + drift).to(inp.k.dtype))
    # The claim above, counted on the scores themselves (log2 units, 32-key blocks, the
    # causal limit ignored): how often a block's maximum exceeds everything before it by
    # more than the 2^8 bound of the row-sum check.
    q, k = f64(inp.q)[0], f64(inp.k)[0]
    s2 = np.einsum("qhd,khd->hqk", q, k) * w.scale / np.log(2.0)
    blocks = s2[:, :, : (n // 32) * 32].reshape(s2.shape[0], s2.shape[1], -1, 32).max(axis=3)
    before = np.maximum.accumulate(blocks, axis=2)[:, :, :-1]
    assert np.mean(blocks[:, :, 1:] - before > 8.0) > 0.5
    o, lse, _, _, _ = run_gpu(inp, causal, w.scale)
    o_ref, lse_ref = oracle.forward(inp.q, inp.k, inp.v, w.scale, causal)
    check(f"growing d{d} c{int(causal)} O", "bf16", o, o_ref, "o")
    check(f"growing d{d} c{int(causal)} LSE", "bf16", lse, lse_ref, "lse")


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys(causal):
    """All keys equal: uniform weights, O is the (prefix) mean of V. The exact dQ is
    zero (dQ_i = scale * K_0 * sum_j dS_ij and rows of dS sum to zero), so rel-L2 is
    undefined there: dQ is held to an absolute bound instead. Each term of that sum
    carries the bf16 rounding of dS (relative 2^-9), so |dQ_i| stays below
    scale * |K_0|_inf * 2^-9 * sum_j |dS_ij|, far under 1e-2 at these sizes."""
    w = _w("bf16", 64, causal)
    inp = W.make_inputs(w, seed=78, batch=1, seqlen=190, heads=1)
    inp.k[:] = inp.k[:, :1]
    o, lse, dq, dk, dv = run_gpu(inp, causal, w.scale)
    o_ref, lse_ref = oracle.forward(inp.q, inp.k, inp.v, w.scale, causal)
    dq_r, dk_r, dv_r = oracle.backward(inp.q, inp.k, inp.v, inp.do, w.scale, causal)
    assert np.abs(dq_r).max() < 1e-12
    check("identical keys O", "bf16", o, o_ref, "o")
    check("identical keys LSE", "bf16", lse, lse_ref, "lse")
    check("identical keys dK", "bf16", dk, dk_r, "g")
    check("identical keys dV", "bf16", dv, dv_r, "g")
    assert f64(dq).__abs__().max() <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bitwise_deterministic(dtype):
    """Forward and backward are bitwise identical from run to run (no atomics)."""
    w = _w(dtype, 128, True)
    inp = W.make_inputs(w, seed=79, batch=2, seqlen=333, heads=2)
    a = run_gpu(inp, True, w.scale)
    b = run_gpu(inp, True, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_outputs_stay_in_bounds():
    """Canary words around every output buffer and the workspace stay untouched."""
    import exact_io_aware_attention_amd as fa
    w = _w("bf16", 128, True)
    B, N, H, d = 1, 321, 3, 128
    inp = W.make_inputs(w, seed=80, batch=B, seqlen=N, heads=H)
    dev = "cuda"
    pad = 4096
    n = B * N * H * d

    def guarded(numel, dtype, fill):
        buf = torch.full((numel + 2 * pad,), fill, device=dev, dtype=dtype)
        return buf, buf[pad:pad + numel]

    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.do))
    ob, o = guarded(n, torch.bfloat16, -1000.0)
    lb, lse = guarded(B * H * N, torch.float32, -1000.0)
    o, lse = o.view(B, N, H, d), lse.view(B, H, N)
    fa.forward(q, k, v, causal=True, softmax_scale=w.scale, out=o, lse=lse)
    grads = [guarded(n, torch.bfloat16, -1000.0) for _ in range(3)]
    dq, dk, dv = (x[1].view(B, N, H, d) for x in grads)
    wsb, ws = guarded(fa.fa_bwd_workspace_bytes(B, H, N, d, 0, 0), torch.uint8, 0xA5)
    fa.backward(q, k, v, o, lse, do, causal=True, softmax_scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for buf, fill in [(ob, -1000.0), (lb, -1000.0), (wsb, 0xA5)] + [(x[0], -1000.0) for x in grads]:
        edges = torch.cat([buf[:pad], buf[-pad:]]).float().cpu().numpy()
        assert np.all(edges == fill)


def test_calls_run_on_the_given_stream():
    """The library enqueues on the caller's stream: work on a side stream, ordered by
    events only, gives the same result as on the default stream."""
    import exact_io_aware_attention_amd as fa
    w = W.get("c3")
    inp = W.make_inputs(w, batch=1, seqlen=300, heads=2)
    q, k, v, do = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.do))
    o0, l0 = fa.forward(q, k, v, causal=True, softmax_scale=w.scale)
    g0 = fa.backward(q, k, v, o0, l0, do, causal=True, softmax_scale=w.scale)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = fa.forward(q, k, v, causal=True, softmax_scale=w.scale, stream=side)
        g1 = fa.backward(q, k, v, o1, l1, do, causal=True, softmax_scale=w.scale, stream=side)
        done = torch.cuda.Event()
        done.record(side)
    done.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
