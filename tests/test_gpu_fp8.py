"""The forward pass on E4M3 inputs (fa_fwd_fp8) against the oracle's exact attention of
the real (decoded, descaled) inputs. Tolerances (parity_utils, "fp8"): O rel-L2 <= 5e-2
and max-abs <= 1e-1 (P is rounded to E4M3 before P V), LSE abs <= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import check

pytestmark = pytest.mark.gpu


def _run(q8, k8, v8, w, causal, scale):
    import exact_io_aware_attention_amd as fa
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), w.descale_q, w.descale_k, w.descale_v,
                            causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 64, 300, 513])
def test_fp8_forward_matches_oracle(d, causal, n):
    w = W.Fp8Workload("t", 2, 2, n, d, causal, 1.0, 3100 + n + d, descale_q=0.5, descale_k=2.0, descale_v=0.75)
    q8, k8, v8 = W.make_fp8_inputs(w)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q8, k8, v8, w, causal, scale)
    o_r, l_r = oracle.forward_fp8(q8.numpy(), k8.numpy(), v8.numpy(), w.descale_q, w.descale_k, w.descale_v,
                                  scale, causal)
    tag = f"fp8 d={d} causal={causal} n={n}"
    for b in range(2):
        for h in range(2):
            check(f"{tag} b{b} h{h} O", "fp8", o[b, :, h, :], o_r[b, :, h, :], "o")
            check(f"{tag} b{b} h{h} LSE", "fp8", lse[b, h, :], l_r[b, h, :], "lse")


def test_fp8_forward_full_workload_sampled_rows():
    """f1 at full size (B=4, H=32, N=4096, d=128, causal), in the launch configuration the
    benchmark times: 24 sampled query rows of every fourth (sequence, head) pair against
    the oracle's rows (the last row and row 0 always among them)."""
    w = W.FP8_WORKLOADS["f1"]
    q8, k8, v8 = W.make_fp8_inputs(w)
    o, lse = _run(q8, k8, v8, w, w.causal, w.scale)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.seqlen - 1], rng.choice(w.seqlen, 22, replace=False)]))
    dec = oracle.e4m3_decode
    for bh in range(0, w.batch * w.heads, 4):
        b, h = divmod(bh, w.heads)
        qh = dec(q8[b, :, h, :].numpy()) * w.descale_q
        kh = dec(k8[b, :, h, :].numpy()) * w.descale_k
        vh = dec(v8[b, :, h, :].numpy()) * w.descale_v
        o_r, l_r = oracle.forward_rows(qh, kh, vh, w.scale, w.causal, rows)
        check(f"f1 b{b} h{h} O rows", "fp8", o[b, rows, h, :], o_r, "o")
        check(f"f1 b{b} h{h} LSE rows", "fp8", lse[b, h, rows], l_r, "lse")


def test_fp8_forward_agrees_with_bf16_forward_on_exact_inputs():
    """Codes whose real values are bf16-exact: the bf16 forward on those values and the
    fp8 forward differ only by the E4M3 rounding of P."""
    import exact_io_aware_attention_amd as fa
    w = W.Fp8Workload("t", 1, 4, 700, 128, True, 1.0, 3200, descale_q=1.0, descale_k=1.0, descale_v=1.0)
    q8, k8, v8 = W.make_fp8_inputs(w)
    dec = lambda t: torch.from_numpy(oracle.e4m3_decode(t.numpy())).to(torch.bfloat16).cuda()
    o_b, l_b = fa.forward(dec(q8), dec(k8), dec(v8), causal=True, softmax_scale=w.scale)
    o_8, l_8 = _run(q8, k8, v8, w, True, w.scale)
    torch.cuda.synchronize()
    assert (l_b.cpu() - l_8).abs().max().item() <= 1e-3
    diff = (o_b.cpu().double() - o_8.double())
    assert diff.norm().item() / o_b.cpu().double().norm().item() <= 5e-2
