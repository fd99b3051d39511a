"""Plain fp64 definition of the gradients of exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

Source: the forward is the one of oracle.attention ("flash attention v3
paper" search-result page, standard self-attention: S = Q K^T, row softmax
P, O = P V; scale after the product as in the "Flash Attention 2 algorithm"
pseudocode of "Flash Attention on the 5090 in CUDA C++"). The pages name the
backward pass and training use ("Flash Attention", aiunderstanding.org) but
print no algorithm for it, so this is the chain rule through that definition
written out, with dO the gradient of a scalar loss with respect to O:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),   D_i = sum_j P_ij dP_ij   (the softmax Jacobian;
                                                   D_i also equals dO_i . O_i)
    dQ = dS K * scale
    dK = dS^T Q * scale

Masked scores have P = 0 and so contribute nothing; a query row without a
visible key has P = 0, hence dQ_i = 0. With GQA (query head h reads KV head
h // (Hq / Hkv)), dK and dV of a KV head are the sums over its query heads.
"""
from __future__ import annotations

import numpy as np

from .attention import _check

NEG_INF = -np.inf


def attention_backward_head(q, k, v, do, scale, causal=False):
    """One query head: q, do [Nq, d], k, v [Nk, d] (its KV head). Returns
    (dQ [Nq,d], dK [Nk,d], dV [Nk,d], D [Nq], P [Nq,Nk], dP [Nq,Nk]), the
    head's contributions to dK and dV before any GQA sum, and the exact
    probabilities and dP = dO V^T they come from. All float64."""
    Nq, Nk = q.shape[0], k.shape[0]
    s = (q @ k.T) * scale
    if causal:
        last = np.arange(Nq) + (Nk - Nq)
        s[np.arange(Nk)[None, :] > last[:, None]] = NEG_INF
    m = s.max(axis=1) if Nk else np.full(Nq, NEG_INF)
    alive = np.isfinite(m)
    e = np.exp(s - np.where(alive, m, 0.0)[:, None])
    p = np.zeros_like(e)
    p[alive] = e[alive] / e[alive].sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    dq = ds @ k * scale
    dk = ds.T @ q * scale
    return dq, dk, dv, dsum, p, dp


def attention_backward(q, k, v, do, scale, causal=False):
    """Gradients (dQ [B,Hq,Nq,d], dK [B,Hkv,Nk,d], dV [B,Hkv,Nk,d]) of the
    loss whose gradient with respect to O = attention(q, k, v) is `do`.
    Also returns D [B,Hq,Nq] = rowsum(P * dP). All float64."""
    B, Hq, Hkv, Nk, d = _check(q, k, v)
    Nq = q.shape[2]
    group = Hq // Hkv
    dq = np.zeros((B, Hq, Nq, d))
    dk = np.zeros((B, Hkv, Nk, d))
    dv = np.zeros((B, Hkv, Nk, d))
    dd = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            dq_h, dk_h, dv_h, dsum, _, _ = attention_backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale,
                                                                   causal)
            dq[b, h] = dq_h
            dk[b, g] += dk_h
            dv[b, g] += dv_h
            dd[b, h] = dsum
    return dq, dk, dv, dd
