"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a flipped comparison, a dropped term, a wrong sign, a
transposed operand) in a private copy of the oracle's source, loads that copy as a
separate module, and checks that at least one pin rejects it. The real oracle is
never modified; the same pins must accept it.
"""
import importlib.util
import itertools
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention.py")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token.json")

MUTATIONS = {
    "causal_mask_off_by_one": ("np.arange(n_k)[None, :] > np.arange(n_q)[:, None]",
                               "np.arange(n_k)[None, :] >= np.arange(n_q)[:, None]"),
    "causal_mask_transposed": ("np.arange(n_k)[None, :] > np.arange(n_q)[:, None]",
                               "np.arange(n_k)[None, :] < np.arange(n_q)[:, None]"),
    "lse_sign": ("m_safe[:, 0] + np.log(", "m_safe[:, 0] - np.log("),
    "max_wrong_axis": ("m = s.max(axis=1, keepdims=True)", "m = s.max(axis=0, keepdims=True)"),
    "dv_not_transposed": ("dv = p.T @ do", "dv = p @ do"),
    "ds_drops_d_term": ("ds = p * (dp - d_row)", "ds = p * dp"),
    "ds_wrong_sign": ("ds = p * (dp - d_row)", "ds = p * (d_row - dp)"),
    "dq_drops_scale": ("dq = scale * (ds @ k)", "dq = (ds @ k)"),
    "dk_wrong_operand": ("dk = scale * (ds.T @ q)", "dk = scale * (ds.T @ k)"),
    "dk_not_transposed": ("dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    "d_row_wrong_axis": ("d_row = (p * dp).sum(axis=1, keepdims=True)",
                         "d_row = (p * dp).sum(axis=0, keepdims=True)"),
    "scores_unscaled": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "rows_mask_off_by_one": ("> np.asarray(rows)[:, None]", ">= np.asarray(rows)[:, None]"),
    "key_rows_d_from_do": ("d_row = (do[rows] * o_rows)", "d_row = (do[rows] * do[rows])"),
    "key_rows_dk_unscaled": ("dk += scale * (ds_sel.T @ q[rows])", "dk += (ds_sel.T @ q[rows])"),
    "packed_lse_layout": ("lse[h, t0:t1] = lh", "lse[h, t0:t1] = lh[::-1]"),
    "decode_top_left_alignment": ("last_visible = n_k - n_q + np.arange(n_q)", "last_visible = np.arange(n_q)"),
    "decode_mask_off_by_one": ("np.arange(n_k)[None, :] > last_visible[:, None]",
                               "np.arange(n_k)[None, :] >= last_visible[:, None]"),
    "decode_lse_layout": ("o[b, :, h, :], lse[b, h, :] = head_decode", "lse[b, h, :], o[b, :, h, :] = head_decode"),
    "stats_padded_layout": ("d_tok.transpose(0, 2, 1) if", "d_tok.transpose(0, 1, 2) if"),
    "stats_packed_layout": ("if cu_seqlens is None else d_tok.T", "if cu_seqlens is None else d_tok"),
    "stats_mneg_sign": ("return d_row, -lse / scale", "return d_row, lse / scale"),
    "stats_mneg_times_scale": ("return d_row, -lse / scale", "return d_row, -lse * scale"),
    "stats_d_from_o_only": ("d_tok = (o * do).sum(axis=-1)", "d_tok = (o * o).sum(axis=-1)"),
}


def _load(source: str, name: str) -> types.ModuleType:
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(source, name, "exec"), mod.__dict__)
    return mod


def _eval(x):
    if isinstance(x, str):
        return eval(x, {"ln2": math.log(2.0), "ln3": math.log(3.0)})
    return float(x)


def _pins(m):
    """Run a compact selection of the oracle pins against module ``m``; return the
    names of those that fail (an exception counts as a failure)."""
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                fn()
        except Exception:
            failed.append(name)

    g = json.load(open(GOLDEN))

    def golden():
        q, k, v, do = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "do"))
        for causal in (False, True):
            e = g["causal" if causal else "noncausal"]
            o, lse = m.head_forward(q, k, v, math.log(2.0), causal)
            np.testing.assert_allclose(o, [[_eval(x) for x in r] for r in e["o"]], atol=1e-12)
            np.testing.assert_allclose(lse, [_eval(x) for x in e["lse"]], atol=1e-12)
            got = m.head_backward(q, k, v, do, math.log(2.0), causal)
            for name, arr in zip(("dq", "dk", "dv"), got):
                np.testing.assert_allclose(arr, [[_eval(x) for x in r] for r in e[name]], atol=1e-12)

    def torch_ref():
        rng = np.random.default_rng(1)
        B, n, H, d = 1, 9, 2, 5
        q, k, v, do = (rng.standard_normal((B, n, H, d)) for _ in range(4))
        for causal in (False, True):
            tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
                          for x in (q, k, v))
            to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.4)
            to.backward(torch.tensor(do).permute(0, 2, 1, 3))
            o, lse = m.forward(q, k, v, 0.4, causal)
            np.testing.assert_allclose(o, to.detach().permute(0, 2, 1, 3).numpy(), atol=1e-10)
            _, tl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
                tq.detach(), tk.detach(), tv.detach(), 0.0, causal, scale=0.4)[:2]
            np.testing.assert_allclose(lse, tl.numpy(), atol=1e-10)
            for mine, t in zip(m.backward(q, k, v, do, 0.4, causal), (tq, tk, tv)):
                np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-10)

    def finite_differences():
        rng = np.random.default_rng(2)
        n, d = 4, 3
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        for causal in (False, True):
            grads = m.head_backward(q, k, v, do, 0.7, causal)
            for which, grad in enumerate(grads):
                for idx in itertools.product(range(n), range(d)):
                    a = [q.copy(), k.copy(), v.copy()]
                    b = [q.copy(), k.copy(), v.copy()]
                    a[which][idx] += 1e-6
                    b[which][idx] -= 1e-6
                    fa = np.sum(m.head_forward(*a, 0.7, causal)[0] * do)
                    fb = np.sum(m.head_forward(*b, 0.7, causal)[0] * do)
                    assert abs(grad[idx] - (fa - fb) / 2e-6) < 1e-6

    def row_helpers():
        rng = np.random.default_rng(3)
        n, d = 40, 4
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        rows = np.array([0, 5, 39])
        for causal in (False, True):
            o, lse = m.head_forward(q, k, v, 0.5, causal)
            dq, dk, dv = m.head_backward(q, k, v, do, 0.5, causal)
            o_r, l_r = m.forward_rows(q, k, v, 0.5, causal, rows)
            np.testing.assert_allclose(o_r, o[rows], atol=1e-12)
            np.testing.assert_allclose(l_r, lse[rows], atol=1e-12)
            np.testing.assert_allclose(m.backward_query_rows(q, k, v, do, 0.5, causal, rows),
                                       dq[rows], atol=1e-12)
            dk_r, dv_r = m.backward_key_rows(q, k, v, do, 0.5, causal, rows, chunk=16)
            np.testing.assert_allclose(dk_r, dk[rows], atol=1e-12)
            np.testing.assert_allclose(dv_r, dv[rows], atol=1e-12)

    def packed():
        rng = np.random.default_rng(4)
        cu = np.array([0, 3, 10, 12])
        q, k, v = (rng.standard_normal((12, 1, 2)) for _ in range(3))
        o, lse = m.forward(q, k, v, 0.5, True, cu_seqlens=cu)
        for s in range(3):
            a, b = cu[s], cu[s + 1]
            oh, lh = m.head_forward(q[a:b, 0], k[a:b, 0], v[a:b, 0], 0.5, True)
            np.testing.assert_allclose(o[a:b, 0], oh, atol=1e-13)
            np.testing.assert_allclose(lse[0, a:b], lh, atol=1e-13)
        # brute force per token
        for t in range(12):
            s = max(i for i in range(3) if cu[i] <= t)
            a = cu[s]
            w = [math.exp(0.5 * float(q[t, 0] @ k[j, 0])) for j in range(a, t + 1)]
            want = sum(wi * v[j, 0] for wi, j in zip(w, range(a, t + 1))) / sum(w)
            np.testing.assert_allclose(o[t, 0], want, atol=1e-12)
            np.testing.assert_allclose(lse[0, t], math.log(sum(w)), atol=1e-12)

    def decode():
        rng = np.random.default_rng(5)
        B, n_q, n_k, H, d = 1, 3, 11, 2, 4
        q, k, v = (rng.standard_normal((B, n, H, d)) for n in (n_q, n_k, n_k))
        for causal in (False, True):
            o, lse = m.decode(q, k, v, 0.6, causal)
            for h in range(H):
                tq, tk, tv = (torch.tensor(x[0, :, h])[None, None] for x in (q, k, v))
                allowed = torch.arange(n_k)[None, :] <= (n_k - n_q + torch.arange(n_q))[:, None]
                mask = allowed[None, None] if causal else None
                to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.6)[0, 0]
                np.testing.assert_allclose(o[0, :, h], to.numpy(), atol=1e-12)
                s = 0.6 * tq[0, 0] @ tk[0, 0].T
                if causal:
                    s = s.masked_fill(~allowed, float("-inf"))
                np.testing.assert_allclose(lse[0, h], torch.logsumexp(s, 1).numpy(), atol=1e-12)

    def stats():
        rng = np.random.default_rng(6)
        B, N, H, d = 2, 5, 3, 4
        q, k, v, do = (rng.standard_normal((B, N, H, d)) for _ in range(4))
        o, lse = m.forward(q, k, v, 0.7, True)
        dvec, mneg = m.backward_stats(o, do, lse, 0.7)
        for b, h in itertools.product(range(B), range(H)):
            s = torch.from_numpy(0.7 * q[b, :, h] @ k[b, :, h].T)
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            p = torch.softmax(s, dim=-1).numpy()
            np.testing.assert_allclose(dvec[b, h], (p * (do[b, :, h] @ v[b, :, h].T)).sum(1), atol=1e-12)
            np.testing.assert_allclose(mneg[b, h], -torch.logsumexp(s, 1).numpy() / 0.7, atol=1e-12)
        T = 6
        o, do, lse = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d)), rng.standard_normal((H, T))
        dvec, mneg = m.backward_stats(o, do, lse, 0.5, cu_seqlens=np.array([0, 2, 6]))
        for t, h in itertools.product(range(T), range(H)):
            np.testing.assert_allclose(dvec[h, t], float(o[t, h] @ do[t, h]), atol=1e-12)
            np.testing.assert_allclose(mneg[h, t], -2.0 * lse[h, t], atol=1e-12)

    for name, fn in (("golden", golden), ("torch", torch_ref), ("fd", finite_differences),
                     ("rows", row_helpers), ("packed", packed), ("decode", decode), ("stats", stats)):
        check(name, fn)
    return failed


def test_pins_accept_the_oracle():
    src = open(SRC).read()
    assert _pins(_load(src, "oracle_copy")) == []


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(mutation):
    old, new = MUTATIONS[mutation]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    mutant = _load(src.replace(old, new), "oracle_mutant_" + mutation)
    assert _pins(mutant), f"no pin caught the planted mistake {mutation}"
