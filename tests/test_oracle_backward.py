"""Pins of the backward oracle (CPU only): finite differences of the forward
definition, torch autograd of the same definition in float64, and identities
the softmax Jacobian fixes."""
import numpy as np
import pytest
import torch

import oracle

CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 3, 4, 2, False),
    (1, 2, 1, 4, 3, 3, True),    # Nq > Nk causal: row 0 has no key
    (2, 2, 2, 5, 7, 2, True),
    (1, 4, 2, 3, 5, 4, False),   # GQA
]


def _inputs(B, Hq, Hkv, Nq, Nk, d, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, Nq, d)), r.standard_normal((B, Hkv, Nk, d)),
            r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hq, Nq, d)))


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    q, k, v, do = _inputs(B, Hq, Hkv, Nq, Nk, d)
    scale = 0.7
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal)
        return float(np.sum(o * do))

    h = 1e-6
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v)
            x[idx] = old - h
            lm = loss(q, k, v)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_autograd(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    q, k, v, do = _inputs(B, Hq, Hkv, Nq, Nk, d, seed=1)
    scale = 0.45
    dq, dk, dv, dsum = oracle.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    kk = tk.repeat_interleave(g, dim=1)
    vv = tv.repeat_interleave(g, dim=1)
    s = (tq @ kk.transpose(-1, -2)) * scale
    if causal:
        vis = torch.arange(Nk)[None, :] <= (torch.arange(Nq) + (Nk - Nq))[:, None]
        s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)  # rows with no visible key
    o = p @ vv
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-12, atol=1e-13)
    # D_i = dO_i . O_i
    o_ref, _ = oracle.attention(q, k, v, scale, causal)
    np.testing.assert_allclose(dsum, (do * o_ref).sum(axis=-1), rtol=1e-12, atol=1e-13)


def test_backward_identities():
    q, k, v, do = _inputs(2, 4, 2, 9, 13, 5, seed=2)
    for causal in (False, True):
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.6, causal)
        # Rows of dS sum to zero, so the key gradients of each head sum to zero.
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # Rows of P sum to one (every row has a key here), so dV sums to dO.
        g = do.reshape(2, 2, 2, 9, 5).sum(axis=2)
        np.testing.assert_allclose(dv.sum(axis=2), g.sum(axis=2), rtol=1e-12, atol=1e-12)
    # V = 1: O = 1 whatever the scores, so Q and K get no gradient.
    dq, dk, dv, _ = oracle.attention_backward(q, k, np.ones_like(v), do, 0.6, True)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


def test_backward_row_without_keys():
    q, k, v, do = _inputs(1, 1, 1, 6, 3, 4, seed=3)
    dq, dk, dv, dsum = oracle.attention_backward(q, k, v, do, 0.5, True)
    # Nq - Nk = 3: rows 0..2 see no key.
    assert np.all(dq[0, 0, :3] == 0.0) and np.all(dsum[0, 0, :3] == 0.0)


def test_backward_head_intermediates():
    """attention_backward_head's P and dP: rows of P sum to one (zero for rows
    without keys), P = exp(S - LSE) with attention's LSE, dP = dO V^T, and the
    head's gradients sum to attention_backward's under GQA."""
    rng = np.random.default_rng(11)
    Nq, Nk, d, scale = 7, 5, 6, 0.4
    q, k, v, do = (rng.standard_normal(s) for s in ((Nq, d), (Nk, d), (Nk, d), (Nq, d)))
    for causal in (False, True):
        dq, dk, dv, D, P, dP = oracle.attention_backward_head(q, k, v, do, scale, causal)
        o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal)
        alive = np.isfinite(lse[0, 0])
        assert np.allclose(P.sum(1)[alive], 1.0, atol=1e-14) and np.all(P[~alive] == 0.0)
        s = q @ k.T * scale
        visible = ~(causal & (np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + (Nk - Nq)))
        ref = np.where(visible & alive[:, None], np.exp(s - np.where(alive, lse[0, 0], 0.0)[:, None]), 0.0)
        assert np.allclose(P, ref, rtol=1e-12, atol=0)
        assert np.allclose(dP, do @ v.T, rtol=1e-13, atol=1e-13)
        assert np.allclose(D, (do * o[0, 0]).sum(1), atol=1e-12)
    # GQA: two query heads on one KV head.
    q2, do2 = rng.standard_normal((1, 2, Nq, d)), rng.standard_normal((1, 2, Nq, d))
    full = oracle.attention_backward(q2, k[None, None], v[None, None], do2, scale, True)
    parts = [oracle.attention_backward_head(q2[0, h], k, v, do2[0, h], scale, True) for h in range(2)]
    assert np.allclose(full[1][0, 0], parts[0][1] + parts[1][1], atol=1e-13)
    assert np.allclose(full[2][0, 0], parts[0][2] + parts[1][2], atol=1e-13)
