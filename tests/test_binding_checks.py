"""The Python binding validates every tensor against q's dimensions before it calls the C
ABI (which takes bare pointers and cannot see sizes). These run on the CPU: each call is
rejected before any device memory or kernel is involved."""
import pytest
import torch

import exact_io_aware_attention_amd as fa

B, N, H, D = 2, 64, 4, 64


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_forward_rejects_mismatched_k_v_out_lse():
    q = t(B, N, H, D)
    with pytest.raises(ValueError, match="^k must have shape"):
        fa.forward(q, t(B, N + 1, H, D), t(B, N, H, D))
    with pytest.raises(ValueError, match="^v must have shape"):
        fa.forward(q, t(B, N, H, D), t(B, N, H, 128))
    with pytest.raises(TypeError, match="^k must be torch.bfloat16"):
        fa.forward(q, t(B, N, H, D, dtype=torch.float32), t(B, N, H, D))
    with pytest.raises(ValueError, match="^out must have shape"):
        fa.forward(q, t(B, N, H, D), t(B, N, H, D), out=t(B, N, H, D - 1))
    with pytest.raises(ValueError, match="^lse must have shape"):
        fa.forward(q, t(B, N, H, D), t(B, N, H, D), lse=t(B, N, H, dtype=torch.float32))
    with pytest.raises(TypeError, match="^lse must be torch.float32"):
        fa.forward(q, t(B, N, H, D), t(B, N, H, D), lse=t(B, H, N))


def test_forward_varlen_checks_cu_seqlens_and_lse():
    T = 100
    q = t(T, H, D)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="max_seqlen is required"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=cu)
    with pytest.raises(TypeError, match="^cu_seqlens must be torch.int32"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=cu.long(), max_seqlen=60)
    with pytest.raises(ValueError, match="^lse must have shape \\(4, 100\\)"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=cu, max_seqlen=60, lse=t(2, H, 60, dtype=torch.float32))


def test_backward_rejects_mismatched_tensors():
    q = t(B, N, H, D)
    lse = t(B, H, N, dtype=torch.float32)
    good = dict(k=t(B, N, H, D), v=t(B, N, H, D), o=t(B, N, H, D), lse=lse, dout=t(B, N, H, D))
    for name in ("k", "v", "o", "dout"):
        bad = dict(good)
        bad[name] = t(B, N, H + 1, D)
        with pytest.raises(ValueError, match=f"^{name} must have shape"):
            fa.backward(q, **bad)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError, match=f"^{name} must have shape"):
            fa.backward(q, **good, **{name: t(B, N, H, D // 2)})
    with pytest.raises(ValueError, match="^lse must have shape"):
        fa.backward(q, **dict(good, lse=t(B, N, dtype=torch.float32)))


def test_decode_and_fp8_forward_reject_mismatched_tensors():
    q = t(B, 1, H, D)
    with pytest.raises(ValueError, match="^v must have shape"):
        fa.decode(q, t(B, 256, H, D), t(B, 255, H, D))
    with pytest.raises(ValueError, match="^k must have shape"):
        fa.decode(q, t(B, 256, H + 1, D), t(B, 256, H, D))
    with pytest.raises(ValueError, match="^lse must have shape"):
        fa.decode(q, t(B, 256, H, D), t(B, 256, H, D), lse=t(B, H, 2, dtype=torch.float32))
    q8 = t(B, N, H, D, dtype=torch.uint8)
    with pytest.raises(ValueError, match="^k8 must have shape"):
        fa.forward_fp8(q8, t(B, N, H, 128, dtype=torch.uint8), q8)
    with pytest.raises(TypeError, match="^v8 must be torch.uint8"):
        fa.forward_fp8(q8, q8, t(B, N, H, D))
    with pytest.raises(TypeError, match="^out must be torch.bfloat16"):
        fa.forward_fp8(q8, q8, q8, out=t(B, N, H, D, dtype=torch.float32))


def test_matching_host_tensors_stop_at_the_device_check():
    q = t(B, N, H, D)
    with pytest.raises(ValueError, match="contiguous device tensors"):
        fa.forward(q, t(B, N, H, D), t(B, N, H, D))


@pytest.mark.parametrize("cu,max_seqlen,msg", [
    ([1, 40, 100], 60, "cu_seqlens\\[0\\] must be 0"),
    ([0, 40, 120], 80, "must equal the packed token count 100"),     # would run past the tensors
    ([0, 40, 90], 60, "must equal the packed token count 100"),
    ([0, 70, 100], 60, "longer than max_seqlen = 60"),              # would leave rows unwritten
    ([0, 60, 50, 100], 60, "non-decreasing"),
])
def test_packed_offsets_are_validated(cu, max_seqlen, msg):
    T = 100
    q = t(T, H, D)
    cu_t = torch.tensor(cu, dtype=torch.int32)
    with pytest.raises(ValueError, match=msg):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=cu_t, max_seqlen=max_seqlen)
    nseq = len(cu) - 1
    lse = t(H, T, dtype=torch.float32)
    with pytest.raises(ValueError, match=msg):
        fa.backward(q, t(T, H, D), t(T, H, D), t(T, H, D), lse, t(T, H, D), cu_seqlens=cu_t,
                    max_seqlen=max_seqlen)
    assert nseq >= 2


def test_packed_offsets_check_can_be_skipped_and_max_seqlen_must_be_positive():
    T = 100
    q = t(T, H, D)
    bad = torch.tensor([0, 70, 100], dtype=torch.int32)
    # without the check the call gets as far as the device test (host tensors here)
    with pytest.raises(ValueError, match="contiguous device tensors"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=bad, max_seqlen=60, check_cu=False)
    with pytest.raises(ValueError, match="max_seqlen must be >= 1"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=torch.tensor([0, 100], dtype=torch.int32),
                   max_seqlen=0)
    good = torch.tensor([0, 40, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="contiguous device tensors"):
        fa.forward(q, t(T, H, D), t(T, H, D), cu_seqlens=good, max_seqlen=60)
