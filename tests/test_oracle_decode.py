"""Pins for the oracle's decode function (Nq new queries against Nk cached keys,
bottom-right causal alignment), each against something other than the function itself:
torch's fp64 attention with an explicit mask, a brute-force loop, closed forms, and the
reduction to the self-attention definition when Nq = Nk."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_q,n_k", [(1, 1), (1, 37), (5, 37), (16, 64), (32, 200)])
def test_decode_matches_torch_with_explicit_mask(causal, n_q, n_k):
    rng = np.random.default_rng(7 + n_q * 1000 + n_k)
    d, scale = 16, 0.37
    q, k, v = _rand(rng, n_q, d), _rand(rng, n_k, d), _rand(rng, n_k, d)
    o, lse = oracle.head_decode(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    mask = None
    if causal:
        # allowed[i, j]: key j at or before query i's absolute position n_k - n_q + i
        allowed = torch.arange(n_k)[None, :] <= (n_k - n_q + torch.arange(n_q))[:, None]
        mask = allowed[None, None]
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(o, to, rtol=1e-12, atol=1e-12)
    s = scale * torch.from_numpy(q) @ torch.from_numpy(k).T
    if causal:
        s = s.masked_fill(~allowed, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_decode_brute_force_loop():
    rng = np.random.default_rng(11)
    n_q, n_k, d, scale = 3, 7, 4, 0.5
    q, k, v = _rand(rng, n_q, d), _rand(rng, n_k, d), _rand(rng, n_k, d)
    o, lse = oracle.head_decode(q, k, v, scale, True)
    for i in range(n_q):
        pos = n_k - n_q + i
        w = [math.exp(scale * sum(q[i, t] * k[j, t] for t in range(d))) for j in range(pos + 1)]
        z = sum(w)
        for t in range(d):
            assert abs(o[i, t] - sum(w[j] * v[j, t] for j in range(pos + 1)) / z) < 1e-12
        assert abs(lse[i] - math.log(z)) < 1e-12


def test_single_query_causal_sees_every_key():
    # the newest query sits at the last position: causal masking hides nothing
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 8), _rand(rng, 50, 8), _rand(rng, 50, 8)
    oc, lc = oracle.head_decode(q, k, v, 0.3, True)
    on, ln = oracle.head_decode(q, k, v, 0.3, False)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)


def test_equal_lengths_reduce_to_self_attention():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 20, 8), _rand(rng, 20, 8), _rand(rng, 20, 8)
    for causal in (False, True):
        o1, l1 = oracle.head_decode(q, k, v, 0.4, causal)
        o2, l2 = oracle.head_forward(q, k, v, 0.4, causal)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def test_constant_keys_give_the_mean_of_visible_values():
    rng = np.random.default_rng(9)
    n_q, n_k = 4, 12
    q, v = _rand(rng, n_q, 6), _rand(rng, n_k, 6)
    k = np.tile(_rand(rng, 1, 6), (n_k, 1))
    o, lse = oracle.head_decode(q, k, v, 0.7, True)
    for i in range(n_q):
        pos = n_k - n_q + i
        np.testing.assert_allclose(o[i], v[: pos + 1].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[i], 0.7 * q[i] @ k[0] + math.log(pos + 1), atol=1e-13)


def test_batched_decode_matches_per_head_calls():
    rng = np.random.default_rng(13)
    B, n_q, n_k, H, d = 2, 3, 9, 2, 4
    q, k, v = _rand(rng, B, n_q, H, d), _rand(rng, B, n_k, H, d), _rand(rng, B, n_k, H, d)
    o, lse = oracle.decode(q, k, v, 0.5, True)
    for b in range(B):
        for h in range(H):
            oh, lh = oracle.head_decode(q[b, :, h], k[b, :, h], v[b, :, h], 0.5, True)
            np.testing.assert_array_equal(o[b, :, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
