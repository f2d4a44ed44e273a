"""A NumPy fp64 model of the tiled recurrences the HIP kernels implement.

Forward: Q, K, V split into tiles; per query row a running maximum m and running sum
l are carried across key tiles and the partial output is rescaled when the maximum
moves ("Softmax en línea" and "Tiling" in the AI Atlas summary of the FlashAttention
paper; "Aperçu technique" on aiunderstanding.org). The maximum may be kept stale
until it has grown by more than ``threshold`` (in log2 units): the result stays
exact because O and l always share one reference maximum.

Backward: P is recomputed tile by tile from the saved logsumexp instead of being
stored ("Recalcular en vez de guardar" in the same summary).

This model is a development aid, separate from the oracle and from the library; it
is checked against the oracle to ~1e-12 for random tile sizes, ragged tails and
causal diagonal tiles.
"""
import math

import numpy as np
import pytest

import oracle

LOG2E = 1.0 / math.log(2.0)


def tiled_forward(q, k, v, scale, causal, br, bc, threshold=0.0):
    n, d = q.shape
    c = scale * LOG2E
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(n, i0 + br))
        qi = q[rows]
        m = np.full(len(rows), -np.inf)      # reference maximum of raw scores
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        last = rows[-1] if causal else n - 1
        for j0 in range(0, last + 1, bc):
            cols = np.arange(j0, min(n, j0 + bc))
            s = qi @ k[cols].T                # raw scores; the scale enters through c
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_tile = s.max(axis=1)
            m_new = np.maximum(m, m_tile)
            # keep the stale maximum unless it grew by more than `threshold` (log2 units)
            grow = (m_new - np.where(np.isfinite(m), m, -np.inf)) * c > threshold
            m_use = np.where(grow | ~np.isfinite(m), m_new, m)
            m_safe = np.where(np.isfinite(m_use), m_use, 0.0)
            alpha = np.exp2((np.where(np.isfinite(m), m, -np.inf) - m_safe) * c)
            alpha = np.where(np.isfinite(m), alpha, 0.0)
            p = np.exp2(s * c - (m_safe * c)[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_use
        o[rows] = acc / l[:, None]
        lse[rows] = scale * m + np.log(l)
    return o, lse


def tiled_backward(q, k, v, do, o, lse, scale, causal, br, bc):
    n, d = q.shape
    c = scale * LOG2E
    D = (do * o).sum(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for j0 in range(0, n, bc):                # one "workgroup" per key tile
        cols = np.arange(j0, min(n, j0 + bc))
        first = (j0 // br) * br if causal else 0
        for i0 in range(first, n, br):
            rows = np.arange(i0, min(n, i0 + br))
            s = q[rows] @ k[cols].T
            p = np.exp2(s * c - (lse[rows] * LOG2E)[:, None])
            if causal:
                p = np.where(cols[None, :] > rows[:, None], 0.0, p)
            dv[cols] += p.T @ do[rows]
            dp = do[rows] @ v[cols].T
            ds = p * (dp - D[rows][:, None])
            dk[cols] += ds.T @ q[rows]
            dq[rows] += ds @ k[cols]
    return dq * scale, dk * scale, dv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,br,bc", [(1, 4, 4), (37, 8, 16), (64, 16, 16), (100, 32, 8), (129, 16, 32)])
@pytest.mark.parametrize("threshold", [0.0, 8.0])
def test_tiled_model_equals_oracle(causal, n, br, bc, threshold):
    rng = np.random.default_rng(n * 7 + br)
    d = 16
    q, k, v, do = (rng.standard_normal((n, d)) * 2.0 for _ in range(4))
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = oracle.head_forward(q, k, v, scale, causal)
    o, lse = tiled_forward(q, k, v, scale, causal, br, bc, threshold)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)
    g_ref = oracle.head_backward(q, k, v, do, scale, causal)
    g = tiled_backward(q, k, v, do, o, lse, scale, causal, br, bc)
    for a, b in zip(g, g_ref):
        np.testing.assert_allclose(a, b, atol=1e-11)


# Keys of a 32-key block held by lane half g (the MFMA output layout: row 8(r/4) + 4g +
# r % 4 of register r), whose exponentials form one lane's share of the row sum.
_HALF_KEYS = [np.array([8 * (r // 4) + 4 * g + r % 4 for r in range(16)]) for g in (0, 1)]


def tiled_forward_sumcheck(q, k, v, scale, causal, br, keep=256.0):
    """The forward with one 32-query block per wave: per 32-key block, exponentials under
    the current reference are kept when every lane's share of the row sum is at most
    `keep` (= 2^8) for every row of the wave; otherwise, and while some row of the wave
    has no reference yet but sees a key of the block, the reference moves to the block's
    exact row maximum first. Returns O, LSE and the largest P ever formed."""
    n, d = q.shape
    c = scale * LOG2E
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    p_max = 0.0
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(n, i0 + br))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        for j0 in range(0, n, 32):
            cols = np.arange(j0, j0 + 32)
            valid = cols < n
            s = np.full((len(rows), 32), -np.inf)
            s[:, valid] = q[rows] @ k[cols[valid]].T
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            nb = np.where(np.isfinite(m), -m * c, 0.0)
            with np.errstate(over="ignore", invalid="ignore"):
                p = np.exp2(s * c + nb[:, None])
            shares = np.stack([p[:, h].sum(axis=1) for h in _HALF_KEYS])
            redo = not np.all(shares <= keep)
            redo |= bool(np.any(~np.isfinite(m) & (s.max(axis=1) > -np.inf)))
            if redo:
                m_new = np.maximum(m, s.max(axis=1))
                m_to = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp2((m - m_to) * c), 0.0)
                l, acc, m = alpha * l, alpha[:, None] * acc, m_new
                p = np.exp2(s * c - (m_to * c)[:, None])
            p_max = max(p_max, float(p.max()))
            l = l + p.sum(axis=1)
            acc = acc + p[:, valid] @ v[cols[valid]]
        o[rows] = acc / l[:, None]
        lse[rows] = scale * m + np.log(l)
    return o, lse, p_max


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 31, 64, 97])
@pytest.mark.parametrize("growth", [0.0, 0.6])
def test_sumcheck_model_equals_oracle(causal, n, growth):
    """Exact (to fp64 rounding) with random scores, and with scores that grow along the
    keys (growth > 0: every later block exceeds the reference, so the uncommon path runs
    again and again); no P ever exceeds 2^8."""
    rng = np.random.default_rng(n + int(10 * growth))
    d = 16
    q, k, v = (rng.standard_normal((n, d)) * 2.0 for _ in range(3))
    k = k + growth * np.arange(n)[:, None] * np.sign(q.mean(axis=0))[None, :]
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = oracle.head_forward(q, k, v, scale, causal)
    o, lse, p_max = tiled_forward_sumcheck(q, k, v, scale, causal, br=32)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-10)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-10, rtol=1e-12)
    assert p_max <= 256.0
