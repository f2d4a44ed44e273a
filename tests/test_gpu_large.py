"""Tensors beyond 4 GiB: 2^31 bf16 elements (2^32 bytes) per operand, so element and
byte offsets leave the 32-bit range; the largest head index of the last sequence sits
at the far end. Forward and backward (bf16 at head_dim 64 and 128, fp32), the 8-bit
forward and decoding over a 4 GiB cache, each through the C ABI in the launch
configuration the benchmark uses, checked against the oracle on sampled heads
(always the first and the last (sequence, head) pair) with the usual tolerances.
Inputs are seeded iid normal values generated on the device."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_utils import check

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


def _heads(B, H):
    return [(0, 0), (B - 1, H - 1), (B // 2 + 13 if B > 26 else B // 2, H // 3)]


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,d,H,B", [("bf16", 128, 128, 128), ("bf16", 64, 256, 128), ("fp32", 128, 128, 64)],
                         ids=["bf16-d128", "bf16-d64", "fp32-d128"])
def test_forward_backward_beyond_4gib(dtype, d, H, B):
    import exact_io_aware_attention_amd as fa
    N, causal, scale = 1024, True, 1.0 / math.sqrt(d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shape = (B, N, H, d)
    assert math.prod(shape) * tdt.itemsize >= 1 << 32
    print(f"large {dtype} {shape} causal", flush=True)
    q, k, v, do = W.make_device_tensors(shape, 4, seed=4100 + d, std=0.5, dtype=tdt)
    o, lse = fa.forward(q, k, v, causal=causal, softmax_scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    for b, h in _heads(B, H):
        qh, kh, vh, doh = (_f64(x[b, :, h, :]) for x in (q, k, v, do))
        o_r, l_r = oracle.head_forward(qh, kh, vh, scale, causal)
        dq_r, dk_r, dv_r = oracle.head_backward(qh, kh, vh, doh, scale, causal)
        tag = f"large {dtype} d={d} b{b} h{h}"
        check(f"{tag} O", dtype, o[b, :, h, :], o_r, "o")
        check(f"{tag} LSE", dtype, lse[b, h, :], l_r, "lse")
        check(f"{tag} dQ", dtype, dq[b, :, h, :], dq_r, "g")
        check(f"{tag} dK", dtype, dk[b, :, h, :], dk_r, "g")
        check(f"{tag} dV", dtype, dv[b, :, h, :], dv_r, "g")


def test_fp8_forward_beyond_4gib():
    import exact_io_aware_attention_amd as fa
    B, N, H, d, causal = 128, 1024, 256, 128, True
    scale, ds = 1.0 / math.sqrt(d), (0.5, 2.0, 0.75)
    shape = (B, N, H, d)
    assert math.prod(shape) >= 1 << 32
    print(f"large fp8 {shape} causal", flush=True)
    q8, k8, v8 = (W.make_device_tensors(shape, 1, seed=4300 + i, std=1.0 / s, dtype=torch.uint8)[0]
                  for i, s in enumerate(ds))
    o, lse = fa.forward_fp8(q8, k8, v8, *ds, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(N)
    for b, h in _heads(B, H):
        qh, kh, vh = (oracle.e4m3_decode(x[b, :, h, :].cpu().numpy()) * s for x, s in zip((q8, k8, v8), ds))
        o_r, l_r = oracle.forward_rows(qh, kh, vh, scale, causal, rows)
        check(f"large fp8 b{b} h{h} O", "fp8", o[b, :, h, :], o_r, "o")
        check(f"large fp8 b{b} h{h} LSE", "fp8", lse[b, h, :], l_r, "lse")


def test_decode_cache_beyond_4gib():
    import exact_io_aware_attention_amd as fa
    B, NQ, NK, H, d = 4, 16, 65536, 64, 128
    scale = 1.0 / math.sqrt(d)
    assert B * NK * H * d * 2 >= 1 << 32
    print(f"large decode B={B} nq={NQ} nk={NK} H={H} d={d}", flush=True)
    (q,) = W.make_device_tensors((B, NQ, H, d), 1, seed=4400, std=1.0, dtype=torch.bfloat16)
    k, v = W.make_device_tensors((B, NK, H, d), 2, seed=4401, std=1.0, dtype=torch.bfloat16)
    o, lse = fa.decode(q, k, v, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    for b, h in _heads(B, H):
        o_r, l_r = oracle.head_decode(*(_f64(x[b, :, h, :]) for x in (q, k, v)), scale, True)
        check(f"large decode b{b} h{h} O", "bf16", o[b, :, h, :], o_r, "o")
        check(f"large decode b{b} h{h} LSE", "bf16", lse[b, h, :], l_r, "lse")
