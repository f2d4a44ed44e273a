"""Plain, slow, obviously correct fp64 attention on the CPU (NumPy).

TEST INFRASTRUCTURE ONLY: called by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library.

What is computed, and where the sources say so
----------------------------------------------
Sources (web pages on FlashAttention):

* [AA]  "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
        AI Atlas paper summary (asternodelab.github.io), sections "En pocas palabras"
        and "Ideas clave".
* [SA]  "FlashAttention-2 (PT)", Systems analysis wiki (systems-analysis.ru), intro and
        "Desempenho e eficiência".
* [AU]  "FlashAttention", aiunderstanding.org, sections "Aperçu" and "Plongée profonde".
* [MS]  "Flash Attention", docs.monostate.ai, section "Con Sequence Packing".

FlashAttention computes exactly the attention of the original Transformer, only
reorganised into blocks ([AA] "En pocas palabras"; [AU] "Aperçu", "Plongée profonde";
[SA] intro: full computational identity with standard attention). The oracle is
therefore *standard attention written out*, with the full N x N score matrix
materialised ([AU] "Plongée profonde" describes that matrix; [AA] "Pensar en la E/S"
describes standard attention writing it to memory):

    S   = scale * Q K^T                         (N x N)
    S_ij = -inf  where key j is hidden from query i (causal: j > i)
    m_i = max_j S_ij,   l_i = sum_j exp(S_ij - m_i)
    P   = exp(S - m) / l                        (row softmax)
    O   = P V
    LSE_i = m_i + ln l_i                        (natural log)

Backward, for an upstream gradient dO: the chain rule of the definition above,

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij                      (equals dO_i . O_i)
    dS = P * (dP - D 1^T)
    dQ = scale * dS K
    dK = scale * dS^T Q

Readings (the pages write no formula; these are the plainest readings the rest
supports):

* r1  scale is an explicit argument; the mask is additive -inf.
* r2  causal: query i sees key j iff j <= i (queries and keys share one length, so
      top-left and bottom-right alignment coincide).
* r3  a row with no visible key (impossible for causal self-attention with N >= 1)
      gets O = 0, LSE = -inf and zero gradients.
* r4  the per-row statistic saved by the forward pass is the natural-log
      logsumexp of the scaled, masked scores.
* r5  packed batches ([MS] "Con Sequence Packing"): attention is block-diagonal per
      sequence; causal applies within each sequence.
* r15 decoding (the pages cite faster inference without a formula): Nq new queries
      attend to a cache of Nk keys of which they are the last Nq positions; under
      causal masking query i (0-based) sees key j iff j <= Nk - Nq + i (bottom-right
      alignment; with Nq = Nk this is r2).

Every function here is pinned by tests that do not retype it: closed forms, hand
derived worked values (tests/golden), invariants, central finite differences,
brute-force loops on tiny inputs, and torch's own fp64 attention and autograd.
Parity pinned: all functions below (none is "parity unpinned").
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

Array = np.ndarray


def to_f64(x) -> Array:
    """Exact upcast of a CPU tensor or array (bf16/fp32/fp64) to a float64 array."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    import torch  # local: the oracle itself needs only NumPy
    return x.detach().to("cpu", torch.float64).numpy()


# ----------------------------------------------------------------------------------------
# One head: q, k, v, do are (N, d) float64.
# ----------------------------------------------------------------------------------------

def _scores(q: Array, k: Array, scale: float, causal: bool) -> Array:
    """S = scale * Q K^T with hidden entries set to -inf (readings r1, r2)."""
    s = scale * (q @ k.T)
    if causal:
        n_q, n_k = s.shape
        hidden = np.arange(n_k)[None, :] > np.arange(n_q)[:, None]
        s = np.where(hidden, -np.inf, s)
    return s


def _softmax_rows(s: Array) -> Tuple[Array, Array]:
    """Row softmax of S and its logsumexp (reading r3 for rows with no visible key)."""
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l[:, 0] > 0, m_safe[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)),
                       -np.inf)
    return p, lse


def head_forward(q: Array, k: Array, v: Array, scale: float, causal: bool) -> Tuple[Array, Array]:
    """Standard attention for one head: returns O (N, d) and LSE (N,)."""
    if q.shape[0] == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    p, lse = _softmax_rows(_scores(q, k, scale, causal))
    return p @ v, lse


def head_backward(q: Array, k: Array, v: Array, do: Array, scale: float,
                  causal: bool) -> Tuple[Array, Array, Array]:
    """Gradients (dQ, dK, dV) of sum(O * dO) for one head, by the chain rule."""
    if q.shape[0] == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    p, _ = _softmax_rows(_scores(q, k, scale, causal))
    dv = p.T @ do
    dp = do @ v.T
    d_row = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d_row)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Whole tensors: (B, N, H, d) padded batches, or (T, H, d) packed with cu_seqlens.
# ----------------------------------------------------------------------------------------

def head_decode(q: Array, k: Array, v: Array, scale: float, causal: bool) -> Tuple[Array, Array]:
    """Nq queries against Nk cached keys (reading r15): O (Nq, d) and LSE (Nq,)."""
    n_q, n_k = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        last_visible = n_k - n_q + np.arange(n_q)  # the absolute position of each query
        s = np.where(np.arange(n_k)[None, :] > last_visible[:, None], -np.inf, s)
    p, lse = _softmax_rows(s)
    return p @ v, lse


def decode(q, k, v, scale: float, causal: bool) -> Tuple[Array, Array]:
    """Batched decode: q (B, Nq, H, d), k and v (B, Nk, H, d); O (B, Nq, H, d) and LSE
    (B, H, Nq)."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, n_q, H, _ = q.shape
    o = np.zeros((B, n_q, H, v.shape[-1]))
    lse = np.zeros((B, H, n_q))
    for b in range(B):
        for h in range(H):
            o[b, :, h, :], lse[b, h, :] = head_decode(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], scale, causal)
    return o, lse


def _segments(shape, cu_seqlens) -> Sequence[Tuple[Optional[int], int, int]]:
    """(batch index or None, token start, token end) of each sequence."""
    if cu_seqlens is None:
        B, N = shape[0], shape[1]
        return [(b, 0, N) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    return [(None, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _head_view(x: Array, seg, h: int) -> Array:
    b, t0, t1 = seg
    return x[b, t0:t1, h, :] if b is not None else x[t0:t1, h, :]


def forward(q, k, v, scale: float, causal: bool, cu_seqlens=None) -> Tuple[Array, Array]:
    """O in the input layout and LSE: (B, H, N) for padded batches, (H, T) for packed."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    H = q.shape[-2]
    o = np.zeros(q.shape[:-1] + (v.shape[-1],))
    if cu_seqlens is None:
        lse = np.zeros((q.shape[0], H, q.shape[1]))
    else:
        lse = np.zeros((H, q.shape[0]))
    for seg in _segments(q.shape, cu_seqlens):
        b, t0, t1 = seg
        for h in range(H):
            oh, lh = head_forward(_head_view(q, seg, h), _head_view(k, seg, h),
                                  _head_view(v, seg, h), scale, causal)
            if b is not None:
                o[b, t0:t1, h, :] = oh
                lse[b, h, t0:t1] = lh
            else:
                o[t0:t1, h, :] = oh
                lse[h, t0:t1] = lh
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool,
             cu_seqlens=None) -> Tuple[Array, Array, Array]:
    """(dQ, dK, dV) in the input layout."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    H = q.shape[-2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for seg in _segments(q.shape, cu_seqlens):
        b, t0, t1 = seg
        for h in range(H):
            g = head_backward(_head_view(q, seg, h), _head_view(k, seg, h),
                              _head_view(v, seg, h), _head_view(do, seg, h), scale, causal)
            for dst, val in zip((dq, dk, dv), g):
                if b is not None:
                    dst[b, t0:t1, h, :] = val
                else:
                    dst[t0:t1, h, :] = val
    return dq, dk, dv


def backward_stats(o, do, lse, scale: float, cu_seqlens=None) -> Tuple[Array, Array]:
    """The two per-row statistics the backward starts from, in the LSE layout ((B, H, N)
    padded, (H, T) packed): D_i = sum_k dO_ik O_ik of the O given (reading r6: the
    stored O, not a recomputed one; for the exact O it equals sum_j P_ij dP_ij) and
    -LSE_i / scale."""
    o, do, lse = to_f64(o), to_f64(do), to_f64(lse)
    d_tok = (o * do).sum(axis=-1)                 # (B, N, H) or (T, H)
    d_row = d_tok.transpose(0, 2, 1) if cu_seqlens is None else d_tok.T
    return d_row, -lse / scale


# ----------------------------------------------------------------------------------------
# Selected rows of one head (long sequences): the same definition, evaluated only for
# the rows asked for. q, k, v, do are (N, d) float64; rows/keys are index arrays.
# ----------------------------------------------------------------------------------------

def _rows_softmax(q: Array, k: Array, scale: float, causal: bool, rows: Array):
    s = scale * (q[rows] @ k.T)
    if causal:
        hidden = np.arange(k.shape[0])[None, :] > np.asarray(rows)[:, None]
        s = np.where(hidden, -np.inf, s)
    return _softmax_rows(s)


def forward_rows(q: Array, k: Array, v: Array, scale: float, causal: bool,
                 rows: Array) -> Tuple[Array, Array]:
    """O[rows] and LSE[rows] of one head."""
    p, lse = _rows_softmax(q, k, scale, causal, rows)
    return p @ v, lse


def backward_query_rows(q: Array, k: Array, v: Array, do: Array, scale: float, causal: bool,
                        rows: Array) -> Array:
    """dQ[rows] of one head: dQ_i depends only on row i of P, dP and D."""
    p, _ = _rows_softmax(q, k, scale, causal, rows)
    dp = do[rows] @ v.T
    d_row = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d_row)
    return scale * (ds @ k)


def backward_key_rows(q: Array, k: Array, v: Array, do: Array, scale: float, causal: bool,
                      keys: Array, chunk: int = 1024) -> Tuple[Array, Array]:
    """dK[keys] and dV[keys] of one head.

    dK_j and dV_j are sums over every query row i, and each term needs the whole row
    i of P (for its normaliser and for D_i). The sums are evaluated over groups of
    ``chunk`` query rows at a time so memory stays O(chunk * N)."""
    keys = np.asarray(keys)
    n = q.shape[0]
    dk = np.zeros((keys.size, k.shape[1]))
    dv = np.zeros((keys.size, v.shape[1]))
    for i0 in range(0, n, chunk):
        rows = np.arange(i0, min(n, i0 + chunk))
        p, _ = _rows_softmax(q, k, scale, causal, rows)
        o_rows = p @ v
        d_row = (do[rows] * o_rows).sum(axis=1, keepdims=True)      # D_i = dO_i . O_i
        p_sel = p[:, keys]
        dp_sel = do[rows] @ v[keys].T
        ds_sel = p_sel * (dp_sel - d_row)
        dv += p_sel.T @ do[rows]
        dk += scale * (ds_sel.T @ q[rows])
    return dk, dv
