"""The seeded input recipe: shapes, seeds, rounding and packed lengths."""
import numpy as np
import torch

import workloads as W


def test_five_workloads_have_the_stated_shapes():
    c = W.WORKLOADS
    assert (c["c1"].batch, c["c1"].heads, c["c1"].seqlen, c["c1"].head_dim, c["c1"].dtype) == \
        (1, 1, 128, 64, "fp32")
    assert (c["c2"].batch, c["c2"].heads, c["c2"].seqlen, c["c2"].head_dim) == (8, 16, 2048, 64)
    assert (c["c3"].batch, c["c3"].heads, c["c3"].seqlen, c["c3"].head_dim) == (4, 32, 4096, 128)
    assert c["c3"].causal and c["c3"].std == 0.5
    assert (c["c4"].batch, c["c4"].heads, c["c4"].seqlen, c["c4"].head_dim) == (1, 8, 65536, 64)
    assert c["c5"].varlen and c["c5"].causal and c["c5"].varlen_total == 16384
    assert abs(c["c1"].scale - 1 / 8) < 1e-15


def test_inputs_are_seeded_and_rounded():
    w = W.get("c1")
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for x, y in zip((a.q, a.k, a.v, a.do), (b.q, b.k, b.v, b.do)):
        assert torch.equal(x, y)
    assert a.q.dtype == torch.float32 and a.q.shape == (1, 128, 1, 64)
    assert not torch.equal(a.q, a.k)
    small = W.make_inputs(W.get("c3"), batch=1, seqlen=64, heads=2)
    assert small.q.dtype == torch.bfloat16 and small.q.shape == (1, 64, 2, 128)
    # N(0,1)*0.5 before rounding
    assert 0.4 < float(small.q.float().std()) < 0.6


def test_packed_lengths():
    w = W.get("c5")
    lengths = W.varlen_lengths(w.seed, w.varlen_total, w.varlen_lo, w.varlen_hi)
    assert sum(lengths) == 16384
    assert all(128 <= n <= 2048 for n in lengths[:-1]) and 1 <= lengths[-1] <= 2048
    inp = W.make_inputs(w)
    assert inp.q.shape == (16384, 32, 128)
    cu = inp.cu_seqlens
    assert cu.dtype == torch.int32 and int(cu[0]) == 0 and int(cu[-1]) == 16384
    assert inp.batch == len(lengths) and inp.seqlen == max(lengths)
    assert np.all(np.diff(cu.numpy()) == np.array(lengths))


def test_sample_rows():
    r = W.sample_rows(7, 65536, 256)
    assert len(r) == 256 and len(set(r.tolist())) == 256 and np.all(np.diff(r) > 0)
    assert np.array_equal(r, W.sample_rows(7, 65536, 256))


def test_device_tensors_are_seeded_and_rounded():
    """make_device_tensors (used for multi-GiB inputs): same seed, same values; tensor i
    uses seed + i; values are the fp32 normals times std rounded to the storage dtype
    (E4M3 codes for uint8)."""
    a1, b1 = W.make_device_tensors((4, 300, 3, 8), 2, seed=9, std=0.5, dtype=torch.bfloat16, device="cpu")
    a2, = W.make_device_tensors((4, 300, 3, 8), 1, seed=9, std=0.5, dtype=torch.bfloat16, device="cpu")
    b2, = W.make_device_tensors((4, 300, 3, 8), 1, seed=10, std=0.5, dtype=torch.bfloat16, device="cpu")
    assert a1.dtype == torch.bfloat16 and a1.shape == (4, 300, 3, 8)
    assert torch.equal(a1, a2) and torch.equal(b1, b2) and not torch.equal(a1, b1)
    g = torch.Generator(device="cpu").manual_seed(9)
    ref = (torch.randn(a1.numel(), generator=g, dtype=torch.float32) * 0.5).to(torch.bfloat16)
    assert torch.equal(a1.flatten(), ref)
    c, = W.make_device_tensors((1000,), 1, seed=3, std=2.0, dtype=torch.uint8, device="cpu")
    g = torch.Generator(device="cpu").manual_seed(3)
    ref8 = (torch.randn(1000, generator=g, dtype=torch.float32) * 2.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert c.dtype == torch.uint8 and torch.equal(c, ref8)
