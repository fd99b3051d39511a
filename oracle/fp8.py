"""Plain fp64 definition of attention over 8-bit floating-point inputs.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

Sources (web pages; cited by title and section):

* "Flash Attention on the 5090 in CUDA C++" (Hacker News digest): the goal
  stated at the top (a hand-written attention kernel so that MXFP8 / NVFP4
  matrix instructions can be used) and "What next" (use NVFP4 / MXFP8 MMA).
* "Flash Attention" (aiunderstanding.org), FAQ: FlashAttention-3 explores
  hardware-specific low-precision paths.

The pages name 8-bit inputs but fix no format, scaling or layout.  Reading
taken (listed with the other readings in the design notes): Q, K and V are
stored as OCP E4M3 bytes with one fp32 descale factor per tensor; the value a
byte stands for is decode(byte) * descale.  The attention itself is the same
exact definition as for bf16 inputs, evaluated in fp64 on those values, so
this module only decodes and then calls :func:`oracle.attention.attention`.
"""
from __future__ import annotations

import numpy as np

from .attention import _check, attention

NEG_INF = -np.inf


def e4m3_value(code: int) -> float:
    """The value of one OCP E4M3 byte, from the format's definition:
    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0 is
    subnormal (mantissa/8 * 2^-6); exponent 15 with mantissa 7 is NaN (the
    format has no infinities, so 0x7E = 1.75 * 2^8 = 448 is the largest)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Exact fp64 values of an array of E4M3 bytes (uint8)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def attention_fp8(q8, k8, v8, descale, scale, causal=False, **kw):
    """Exact attention of the values the fp8 inputs stand for:
    Q = decode(q8) * descale[0], K = decode(k8) * descale[1],
    V = decode(v8) * descale[2]; then O = softmax(Q K^T * scale) V with LSE,
    as :func:`oracle.attention.attention` (same keyword arguments)."""
    q = e4m3_decode(q8) * float(descale[0])
    k = e4m3_decode(k8) * float(descale[1])
    v = e4m3_decode(v8) * float(descale[2])
    return attention(q, k, v, scale, causal, **kw)


def prob_weighted_abs(q, k, v, scale, causal=False, q_index=None, nq=None):
    """Two quantities of the exact probabilities P = softmax(Q K^T * scale)
    (same mask and GQA reading as :func:`oracle.attention.attention`), used to
    bound how rounding P before P.V moves O:
      W[b, h, i, :] = sum_j P_ij |V_j|   (elementwise absolute value of V rows)
      Pmax[b, h, i] = max_j P_ij
    Rows with no visible key give W = 0 and Pmax = 0."""
    B, Hq, Hkv, Nk, d = _check(q, k, v)
    n = q.shape[2]
    group = Hq // Hkv
    q_index = np.arange(n) if q_index is None else np.asarray(q_index)
    nq = n if nq is None else nq
    w = np.zeros((B, Hq, n, d))
    pmax = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = (q[b, h] @ k[b, g].T) * scale
            if causal:
                last = q_index + (Nk - nq)
                s[np.arange(Nk)[None, :] > last[:, None]] = NEG_INF
            m = s.max(axis=1) if Nk else np.full(n, NEG_INF)
            alive = np.isfinite(m)
            e = np.exp(s - np.where(alive, m, 0.0)[:, None])
            p = np.zeros_like(e)
            p[alive] = e[alive] / e[alive].sum(axis=1, keepdims=True)
            w[b, h] = p @ np.abs(v[b, g])
            pmax[b, h] = p.max(axis=1) if Nk else 0.0
    return w, pmax
