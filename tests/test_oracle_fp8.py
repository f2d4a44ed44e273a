"""Pins of the E4M3 decoder and the FP8-input forward of the oracle (CPU only).

The decoder is checked against the format's own constants (largest finite value 448,
smallest normal 2^-6, smallest subnormal 2^-9, NaN codes, signed zero), its grid and
ordering, and against torch's float8_e4m3fn conversion of all 256 codes; the forward
against closed forms and a brute-force loop over hand-decoded codes.
"""
import math

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, forward_fp8



def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_decode_format_constants():
    d = lambda c: float(e4m3_decode(np.array([c], dtype=np.uint8))[0])
    assert d(0x00) == 0.0 and not math.copysign(1.0, d(0x00)) < 0
    assert d(0x80) == 0.0 and math.copysign(1.0, d(0x80)) < 0
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0      # largest finite magnitude
    assert d(0x08) == 2.0 ** -6                          # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals
    assert d(0x40) == 2.0 and d(0x3C) == 1.5 and d(0x2A) == 0.3125
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x77) == 240.0 and d(0x78) == 256.0


def test_decode_grid_order_and_sign():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))          # 0x00 .. 0x7E
    assert np.all(np.diff(pos) > 0)                              # strictly increasing
    assert np.all(pos * 2 ** 9 == np.round(pos * 2 ** 9))        # on the 2^-9 grid
    neg = e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)
    assert np.isnan(e4m3_decode(np.arange(256, dtype=np.uint8))).sum() == 2


def _codes(values):
    """Hand table of exact E4M3 codes (sign, exponent field, mantissa field)."""
    table = {0.0: 0x00, 1.0: 0x38, -1.0: 0xB8, 2.0: 0x40, -2.0: 0xC0, 0.5: 0x30, -0.5: 0xB0, 1.5: 0x3C,
             3.0: 0x44, 0.25: 0x28}
    return np.vectorize(lambda v: table[v])(np.asarray(values, dtype=np.float64)).astype(np.uint8)


def test_forward_fp8_equal_keys_closed_form():
    # every key row equal: each query's scores are one constant, softmax is uniform
    N, d = 6, 4
    rng = np.random.default_rng(0)
    vals = [0.0, 1.0, -1.0, 2.0, 0.5, -0.5, 1.5]
    qv = rng.choice(vals, size=(1, N, 1, d))
    kv = np.tile(rng.choice(vals, size=(1, 1, 1, d)), (1, N, 1, 1))
    vv = rng.choice(vals, size=(1, N, 1, d))
    dq, dk, dv, scale = 0.5, 2.0, 0.25, 0.7
    for causal in (False, True):
        o, lse = forward_fp8(_codes(qv), _codes(kv), _codes(vv), dq, dk, dv, scale, causal)
        for i in range(N):
            n = i + 1 if causal else N
            s = scale * dq * dk * float(qv[0, i, 0] @ kv[0, 0, 0])
            np.testing.assert_allclose(o[0, i, 0], dv * vv[0, :n, 0].mean(axis=0), rtol=0, atol=1e-15)
            np.testing.assert_allclose(lse[0, 0, i], s + math.log(n), rtol=0, atol=1e-12)


def test_forward_fp8_brute_force():
    rng = np.random.default_rng(1)
    B, N, H, d = 2, 5, 2, 4
    vals = [0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, 1.5, 3.0, 0.25]
    qv, kv, vv = (rng.choice(vals, size=(B, N, H, d)) for _ in range(3))
    dq, dk, dv, scale = 0.75, 0.5, 2.0, 0.9
    for causal in (False, True):
        o, lse = forward_fp8(_codes(qv), _codes(kv), _codes(vv), dq, dk, dv, scale, causal)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    keys = range(i + 1) if causal else range(N)
                    s = [scale * sum(dq * qv[b, i, h, t] * dk * kv[b, j, h, t] for t in range(d)) for j in keys]
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    tot = sum(w)
                    for t in range(d):
                        ref = sum(wj * dv * vv[b, j, h, t] for wj, j in zip(w, keys)) / tot
                        assert abs(o[b, i, h, t] - ref) < 1e-12
                    assert abs(lse[b, h, i] - (m + math.log(tot))) < 1e-12
