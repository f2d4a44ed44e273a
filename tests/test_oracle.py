"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-derived worked values (tests/golden/two_token.json),
* closed forms (N = 1, scale = 0, constant keys, Q = 0, causal row 0),
* invariants (rows of P sum to one, key/value permutation, key shift, gradient sums),
* central finite differences of the loss sum(O * dO),
* brute-force pure-Python loops on tiny inputs,
* torch's own fp64 CPU attention (forward, logsumexp, and autograd gradients),
* a packed batch equals separate per-sequence calls; selected-row helpers equal the
  full computation.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import varlen_lengths, cu_seqlens_from_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token.json")

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _eval(x):
    if isinstance(x, str):
        return eval(x, {"ln2": math.log(2.0), "ln3": math.log(3.0)})
    return float(x)


def _arr(rows):
    return np.array([[_eval(x) for x in r] for r in rows]) if isinstance(rows[0], list) \
        else np.array([_eval(x) for x in rows])


# ---------------------------------------------------------------- worked example

@pytest.mark.parametrize("causal", [False, True])
def test_golden_two_token(causal):
    g = json.load(open(GOLDEN))
    scale = math.log(2.0)
    q, k, v, do = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "do"))
    exp = g["causal" if causal else "noncausal"]
    o, lse = oracle.head_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, _arr(exp["o"]), atol=1e-15)
    np.testing.assert_allclose(lse, _arr(exp["lse"]), atol=1e-15)
    dq, dk, dv = oracle.head_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, _arr(exp["dq"]), atol=1e-15)
    np.testing.assert_allclose(dk, _arr(exp["dk"]), atol=1e-15)
    np.testing.assert_allclose(dv, _arr(exp["dv"]), atol=1e-15)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_single_token(causal):
    rng = np.random.default_rng(0)
    q, k, v, do = (_rand(rng, 1, 5) for _ in range(4))
    o, lse = oracle.head_forward(q, k, v, 0.7, causal)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, [0.7 * float(q[0] @ k[0])], atol=1e-15)
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.7, causal)
    np.testing.assert_allclose(dv, do, atol=1e-15)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)


def _prefix_mean(v):
    return np.cumsum(v, axis=0) / np.arange(1, v.shape[0] + 1)[:, None]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", ["scale0", "const_k", "zero_q"])
def test_uniform_weights_give_mean_of_v(causal, case):
    rng = np.random.default_rng(1)
    n, d = 9, 4
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    scale = 0.5
    if case == "scale0":
        scale = 0.0
    elif case == "const_k":
        k = np.tile(_rand(rng, 1, d), (n, 1))
    else:
        q = np.zeros((n, d))
    o, lse = oracle.head_forward(q, k, v, scale, causal)
    want = _prefix_mean(v) if causal else np.tile(v.mean(axis=0), (n, 1))
    np.testing.assert_allclose(o, want, atol=1e-13)
    # every visible weight is exp(c) for the same c per row: LSE = c + ln(#visible)
    c = scale * (q @ k[0])
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    np.testing.assert_allclose(lse, c + np.log(cnt), atol=1e-13)


def test_causal_first_row_is_first_value():
    rng = np.random.default_rng(2)
    q, k, v = (_rand(rng, 7, 3) for _ in range(3))
    o, lse = oracle.head_forward(q, k, v, 0.9, True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.9 * q[0] @ k[0], atol=1e-15)


# ---------------------------------------------------------------- invariants

def test_key_value_permutation_invariance_noncausal():
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 11, 6) for _ in range(3))
    perm = rng.permutation(11)
    o1, l1 = oracle.head_forward(q, k, v, 0.4, False)
    o2, l2 = oracle.head_forward(q, k[perm], v[perm], 0.4, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_causal_is_not_permutation_invariant():
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 6, 4) for _ in range(3))
    perm = np.arange(6)[::-1]
    o1, _ = oracle.head_forward(q, k, v, 0.4, True)
    o2, _ = oracle.head_forward(q, k[perm], v[perm], 0.4, True)
    assert np.abs(o1 - o2).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    """K_j -> K_j + u for all j: O unchanged, LSE_i shifts by scale * q_i . u."""
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 10, 5) for _ in range(3))
    u = _rand(rng, 5)
    o1, l1 = oracle.head_forward(q, k, v, 0.3, causal)
    o2, l2 = oracle.head_forward(q, k + u, v, 0.3, causal)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, 0.3 * q @ u, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_normalises_probabilities(causal):
    """exp(S - LSE) rows sum to one (P is a row-stochastic matrix)."""
    rng = np.random.default_rng(5)
    q, k, v = (_rand(rng, 13, 4) for _ in range(3))
    _, lse = oracle.head_forward(q, k, v, 1.1, causal)
    s = 1.1 * q @ k.T
    if causal:
        s[np.triu_indices(13, 1)] = -np.inf
    np.testing.assert_allclose(np.exp(s - lse[:, None]).sum(axis=1), 1.0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    rng = np.random.default_rng(6)
    n, d = 12, 5
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.6, causal)
    # rows of P sum to one => sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # rows of dS sum to zero => sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # tr(Q^T dQ) = tr(K^T dK) = scale * sum(dS * QK^T)
    np.testing.assert_allclose(np.sum(q * dq), np.sum(k * dk), atol=1e-12)


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(causal):
    rng = np.random.default_rng(7)
    n, d, scale = 6, 3, 0.8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    dq, dk, dv = oracle.head_backward(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.head_forward(q_, k_, v_, scale, causal)
        return float(np.sum(o * do))

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in itertools.product(range(n), range(d)):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- brute force

def _brute_force(q, k, v, scale, causal):
    n, d = len(q), len(q[0])
    out, lse = [], []
    for i in range(n):
        vis = [j for j in range(n) if not (causal and j > i)]
        sc = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in vis]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        tot = math.fsum(w)
        out.append([math.fsum(w[a] * v[j][t] for a, j in enumerate(vis)) / tot
                    for t in range(len(v[0]))])
        lse.append(mx + math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("n", [1, 2, 5, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_loops(n, causal):
    rng = np.random.default_rng(8 + n)
    q, k, v = (_rand(rng, n, 3) for _ in range(3))
    o, lse = oracle.head_forward(q, k, v, 0.45, causal)
    ob, lb = _brute_force(q.tolist(), k.tolist(), v.tolist(), 0.45, causal)
    np.testing.assert_allclose(o, ob, atol=1e-14)
    np.testing.assert_allclose(lse, lb, atol=1e-14)


# ---------------------------------------------------------------- torch fp64 attention

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(17, 8), (64, 16), (130, 32)])
def test_matches_torch_fp64_attention(causal, n, d):
    rng = np.random.default_rng(9)
    B, H, scale = 2, 3, 1.0 / math.sqrt(d)
    q, k, v, do = (_rand(rng, B, n, H, d) for _ in range(4))
    o, lse = oracle.forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
                  for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, to.detach().permute(0, 2, 1, 3).numpy(), atol=1e-12)
    _, tlse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq.detach(), tk.detach(), tv.detach(), 0.0, causal, scale=scale)[:2]
    np.testing.assert_allclose(lse, tlse.numpy(), atol=1e-12)
    to.backward(torch.tensor(do).permute(0, 2, 1, 3))
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal)
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11)


# ---------------------------------------------------------------- packing and row helpers

@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_separate_calls(causal):
    lengths = varlen_lengths(3, 200, 5, 60)
    assert sum(lengths) == 200
    cu = cu_seqlens_from_lengths(lengths).numpy()
    rng = np.random.default_rng(10)
    H, d = 2, 4
    q, k, v, do = (_rand(rng, 200, H, d) for _ in range(4))
    o, lse = oracle.forward(q, k, v, 0.5, causal, cu_seqlens=cu)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.5, causal, cu_seqlens=cu)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            oh, lh = oracle.head_forward(q[a:b, h], k[a:b, h], v[a:b, h], 0.5, causal)
            np.testing.assert_allclose(o[a:b, h], oh, atol=1e-15)
            np.testing.assert_allclose(lse[h, a:b], lh, atol=1e-15)
            g = oracle.head_backward(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], 0.5, causal)
            for full, part in zip((dq, dk, dv), g):
                np.testing.assert_allclose(full[a:b, h], part, atol=1e-15)
    # tokens never attend across sequences: changing sequence 0 leaves the others alone
    k2 = k.copy()
    k2[: cu[1]] += 5.0
    o2, _ = oracle.forward(q, k2, v, 0.5, causal, cu_seqlens=cu)
    np.testing.assert_allclose(o2[cu[1]:], o[cu[1]:], atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_row_helpers_equal_full(causal):
    rng = np.random.default_rng(11)
    n, d = 300, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    rows = np.array([0, 1, 17, 128, 255, 299])
    o, lse = oracle.head_forward(q, k, v, 0.35, causal)
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.35, causal)
    orr, lr = oracle.forward_rows(q, k, v, 0.35, causal, rows)
    np.testing.assert_allclose(orr, o[rows], atol=1e-13)
    np.testing.assert_allclose(lr, lse[rows], atol=1e-13)
    np.testing.assert_allclose(oracle.backward_query_rows(q, k, v, do, 0.35, causal, rows),
                               dq[rows], atol=1e-13)
    dkr, dvr = oracle.backward_key_rows(q, k, v, do, 0.35, causal, rows, chunk=64)
    np.testing.assert_allclose(dkr, dk[rows], atol=1e-12)
    np.testing.assert_allclose(dvr, dv[rows], atol=1e-12)


def test_empty_sequence_in_pack():
    cu = np.array([0, 3, 3, 5])
    rng = np.random.default_rng(12)
    q, k, v, do = (_rand(rng, 5, 1, 2) for _ in range(4))
    o, lse = oracle.forward(q, k, v, 1.0, True, cu_seqlens=cu)
    assert o.shape == (5, 1, 2) and np.isfinite(o).all() and np.isfinite(lse).all()


# ---------------------------------------------------------------- backward statistics

@pytest.mark.parametrize("causal", [False, True])
def test_backward_stats_equal_the_softmax_identity(causal):
    """For the exact O, D_i = dO_i . O_i equals sum_j P_ij dP_ij with P from torch's own
    fp64 softmax and dP = dO V^T: a second route to the same number."""
    rng = np.random.default_rng(31)
    B, N, H, d, scale = 2, 9, 3, 5, 0.7
    q, k, v, do = (_rand(rng, B, N, H, d) for _ in range(4))
    o, lse = oracle.forward(q, k, v, scale, causal)
    dvec, mneg = oracle.backward_stats(o, do, lse, scale)
    assert dvec.shape == (B, H, N) and mneg.shape == (B, H, N)
    for b, h in itertools.product(range(B), range(H)):
        s = torch.from_numpy(scale * q[b, :, h] @ k[b, :, h].T)
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        p = torch.softmax(s, dim=-1).numpy()
        dp = do[b, :, h] @ v[b, :, h].T
        np.testing.assert_allclose(dvec[b, h], (p * dp).sum(axis=1), atol=1e-12)
        np.testing.assert_allclose(mneg[b, h], -torch.logsumexp(s, dim=-1).numpy() / scale, atol=1e-12)


def test_backward_stats_layouts_by_loops():
    """Padded (B, H, N) and packed (H, T) layouts against explicit loops, with an O that
    is not an attention output (reading r6: D comes from whatever O is stored)."""
    rng = np.random.default_rng(32)
    B, N, H, d = 2, 4, 3, 2
    o, do = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    lse = _rand(rng, B, H, N)
    dvec, mneg = oracle.backward_stats(o, do, lse, 0.5)
    for b, n, h in itertools.product(range(B), range(N), range(H)):
        assert dvec[b, h, n] == pytest.approx(sum(o[b, n, h, j] * do[b, n, h, j] for j in range(d)), abs=1e-14)
        assert mneg[b, h, n] == pytest.approx(-2.0 * lse[b, h, n], abs=1e-14)
    T = 7
    o, do, lse = _rand(rng, T, H, d), _rand(rng, T, H, d), _rand(rng, H, T)
    dvec, mneg = oracle.backward_stats(o, do, lse, 0.25, cu_seqlens=np.array([0, 3, 7]))
    assert dvec.shape == (H, T)
    for t, h in itertools.product(range(T), range(H)):
        assert dvec[h, t] == pytest.approx(sum(o[t, h, j] * do[t, h, j] for j in range(d)), abs=1e-14)
        assert mneg[h, t] == pytest.approx(-4.0 * lse[h, t], abs=1e-14)
