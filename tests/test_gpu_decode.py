"""Decoding on the GPU (fa_fwd_decode) against the oracle's decode: seqlen_q new
queries against a cache of seqlen_k keys, bottom-right causal alignment, the key range
split and merged by logsumexp. Tolerances are the forward's (bf16 O: max-abs <= 2e-2,
rel-L2 <= 1e-2; LSE diagnostic)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import check

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, scale, num_splits=0):
    import exact_io_aware_attention_amd as fa
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.decode(qd, kd, vd, causal=causal, softmax_scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_all(tag, q, k, v, causal, scale, o, lse):
    o_r, l_r = oracle.decode(q, k, v, scale, causal)
    B, _, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            check(f"{tag} b{b} h{h} O", "bf16", o[b, :, h, :], o_r[b, :, h, :], "o")
            check(f"{tag} b{b} h{h} LSE", "bf16", lse[b, h, :], l_r[b, h, :], "lse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,splits", [(1, 1, 0), (1, 63, 0), (1, 1000, 0), (5, 200, 0), (16, 1500, 3),
                                            (32, 32, 0), (32, 4100, 0), (7, 777, 13), (1, 2048, 1)])
def test_decode_matches_oracle(d, causal, nq, nk, splits):
    w = W.DECODE_WORKLOADS["d2"]
    q, k, v = W.make_decode_inputs(w, seed=11 + nq + nk + d, batch=2, seqlen_q=nq, seqlen_k=nk, heads=3,
                                   head_dim=d)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, causal, scale, splits)
    _check_all(f"decode d={d} causal={causal} nq={nq} nk={nk} splits={splits}", q, k, v, causal, scale, o, lse)


def test_decode_equals_self_attention_when_lengths_match():
    # with seqlen_q == seqlen_k the decode path computes ordinary causal attention
    import exact_io_aware_attention_amd as fa
    w = W.DECODE_WORKLOADS["d2"]
    q, k, v = W.make_decode_inputs(w, seed=5, batch=2, seqlen_q=32, seqlen_k=32, heads=2, head_dim=128)
    o_dec, l_dec = _run(q, k, v, True, 0.1)
    o_fwd, l_fwd = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=True, softmax_scale=0.1)
    torch.cuda.synchronize()
    assert (o_dec.float() - o_fwd.cpu().float()).abs().max().item() <= 2e-2
    assert (l_dec - l_fwd.cpu()).abs().max().item() <= 1e-3


@pytest.mark.parametrize("name", sorted(W.DECODE_WORKLOADS))
def test_decode_workloads_full_size(name):
    """The full decode workloads: every (sequence, head) against the oracle (each is a
    small Nq x Nk product, cheap on the CPU)."""
    w = W.DECODE_WORKLOADS[name]
    q, k, v = W.make_decode_inputs(w)
    o, lse = _run(q, k, v, w.causal, w.scale)
    _check_all(name, q, k, v, w.causal, w.scale, o, lse)


def test_decode_repeated_calls_reuse_the_workspace():
    # the workspace holds no state between calls: a second, smaller call through the
    # same workspace gives its own correct result
    import exact_io_aware_attention_amd as fa
    w = W.DECODE_WORKLOADS["d1"]
    ws = torch.empty(fa.fa_fwd_decode_workspace_bytes(2, 4, 8, 3000, 128, 0), device="cuda", dtype=torch.uint8)
    for nq, nk in ((8, 3000), (3, 900)):
        q, k, v = W.make_decode_inputs(w, seed=nq, batch=2, seqlen_q=nq, seqlen_k=nk, heads=4)
        o, lse = fa.decode(q.cuda(), k.cuda(), v.cuda(), causal=True, softmax_scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        _check_all(f"ws nq={nq} nk={nk}", q, k, v, True, w.scale, o.cpu(), lse.cpu())
