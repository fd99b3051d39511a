"""Checks that pin an attention implementation to facts fixed by the pages and by
mathematics, independent of the implementation under test.

Each ``pin_*`` takes ``attn(q, k, v, scale, causal) -> (O, LSE)`` (float64
numpy arrays, shapes [B, H, N, d]) and raises AssertionError on a mismatch.
They are applied to the oracle (all must pass) and to deliberately wrong
variants of it (each variant must fail at least one), which shows the pins
can tell a plausible mistake from the definition.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-12


def brute_attention(q, k, v, scale, causal):
    """Pure-Python loops with exactly rounded sums (math.fsum): the definition
    softmax(scale * q_i . k_j) over the visible keys, weights applied to V."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    O = np.zeros((B, Hq, Nq, d))
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Nq):
                scores = []
                for j in range(Nk):
                    if causal and j > i + (Nk - Nq):
                        continue
                    dot = math.fsum(float(q[b, h, i, c]) * float(k[b, g, j, c]) for c in range(d))
                    scores.append((j, scale * dot))
                if not scores:
                    continue
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                tot = math.fsum(x for _, x in w)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(x * float(v[b, g, j, c]) for j, x in w) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin_a, fin_b = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fin_a, fin_b), f"{what}: finite pattern differs"
    assert np.array_equal(a[~fin_a], b[~fin_b]), f"{what}: infinities differ"
    if fin_a.any():
        err = np.max(np.abs(a[fin_a] - b[fin_b]) / np.maximum(1.0, np.abs(b[fin_b])))
        assert err <= tol, f"{what}: max rel/abs error {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


# Small shapes that exercise Nq != Nk in both directions, GQA, odd d.
BRUTE_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 5, 5, 3, False),
    (1, 1, 1, 5, 5, 3, True),
    (2, 4, 2, 3, 7, 4, True),
    (1, 2, 1, 7, 3, 2, True),   # Nq > Nk: first rows see no key
    (1, 3, 3, 6, 8, 5, False),
    (1, 2, 2, 1, 6, 4, True),   # decode-like row
]


def pin_brute_force(attn, cases=BRUTE_CASES, seed=1):
    for n, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate(cases):
        r = _rng(seed + n)
        q = r.standard_normal((B, Hq, Nq, d))
        k = r.standard_normal((B, Hkv, Nk, d))
        v = r.standard_normal((B, Hkv, Nk, d))
        scale = 0.5 + r.random()
        O, L = attn(q, k, v, scale, causal)
        Ob, Lb = brute_attention(q, k, v, scale, causal)
        _close(O, Ob, 1e-12, f"brute O case {n}")
        _close(L, Lb, 1e-12, f"brute LSE case {n}")


def pin_identical_keys(attn, seed=2):
    """Every key equal: the weights are uniform, O_i is the column mean of V and
    LSE_i = scale * q_i . k + ln Nk."""
    r = _rng(seed)
    Nq, Nk, d = 6, 9, 4
    q = r.standard_normal((1, 1, Nq, d))
    krow = r.standard_normal(d)
    k = np.broadcast_to(krow, (1, 1, Nk, d)).copy()
    v = r.standard_normal((1, 1, Nk, d))
    scale = 0.75
    O, L = attn(q, k, v, scale, False)
    _close(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (Nq, d)), 1e-13, "identical keys O")
    _close(L[0, 0], scale * (q[0, 0] @ krow) + math.log(Nk), 1e-13, "identical keys LSE")


def pin_one_hot(attn, seed=3):
    """K_j = c * e_j and Q_i = e_{t(i)}: scale * q_i . k_j is c*scale on one key
    and 0 elsewhere, so O_i = (e^{cs} V_t + sum_{j != t} V_j) / (e^{cs} + Nk - 1)
    and LSE_i = cs + ln(1 + (Nk - 1) e^{-cs}).  With cs about 45 the row selects
    V_t."""
    r = _rng(seed)
    Nk = d = 8
    Nq = 5
    c = 400.0
    scale = 0.1125
    cs = c * scale
    t = r.integers(0, Nk, size=Nq)
    q = np.zeros((1, 1, Nq, d))
    q[0, 0, np.arange(Nq), t] = 1.0
    k = (c * np.eye(Nk, d))[None, None]
    v = r.standard_normal((1, 1, Nk, d))
    O, L = attn(q, k, v, scale, False)
    tot = v[0, 0].sum(axis=0)
    for i in range(Nq):
        expect = (math.exp(cs) * v[0, 0, t[i]] + (tot - v[0, 0, t[i]])) / (math.exp(cs) + Nk - 1)
        _close(O[0, 0, i], expect, 1e-13, "one-hot O")
        _close(L[0, 0, i], cs + math.log1p((Nk - 1) * math.exp(-cs)), 1e-13, "one-hot LSE")
        _close(O[0, 0, i], v[0, 0, t[i]], 1e-12, "one-hot selects V_t")


def pin_row_shift(attn, seed=4):
    """K' = K + 1 w^T adds scale * q_i . w to every score of row i: O is
    unchanged and LSE moves by exactly that amount.  A shift of about 900 also
    needs the max subtraction (exp(900) overflows float64)."""
    r = _rng(seed)
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 5, 7, 4
    q = r.standard_normal((B, Hq, Nq, d))
    q[..., 0] = np.abs(q[..., 0]) + 1.0
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    scale = 0.5
    for big in (3.0, 1800.0):
        w = np.zeros(d)
        w[0] = big
        O, L = attn(q, k, v, scale, False)
        O2, L2 = attn(q, k + w, v, scale, False)
        _close(O2, O, 1e-9, f"row shift O ({big})")
        shift = scale * (q @ w)
        _close(L2, L + shift, 1e-12, f"row shift LSE ({big})")


def pin_special_cases(attn, seed=5):
    r = _rng(seed)
    # V = ones => O = 1.
    q = r.standard_normal((1, 2, 4, 3))
    k = r.standard_normal((1, 2, 6, 3))
    O, _ = attn(q, k, np.ones_like(k), 0.7, True)
    _close(O, np.ones_like(O), 1e-14, "V = 1")
    # Nk = 1 => O = V_0, LSE = the single score.
    k1 = r.standard_normal((1, 2, 1, 3))
    v1 = r.standard_normal((1, 2, 1, 3))
    O, L = attn(q, k1, v1, 0.7, False)
    _close(O, np.broadcast_to(v1, O.shape), 1e-14, "Nk = 1 O")
    _close(L, 0.7 * (q @ k1.transpose(0, 1, 3, 2))[..., 0], 1e-14, "Nk = 1 LSE")
    # Causal with Nq == Nk: row 0 sees only key 0; the last row sees all keys.
    qq = r.standard_normal((1, 1, 6, 3))
    kk = r.standard_normal((1, 1, 6, 3))
    vv = r.standard_normal((1, 1, 6, 3))
    O, L = attn(qq, kk, vv, 0.9, True)
    _close(O[0, 0, 0], vv[0, 0, 0], 1e-14, "causal row 0")
    _close(L[0, 0, 0], 0.9 * (qq[0, 0, 0] @ kk[0, 0, 0]), 1e-14, "causal row 0 LSE")
    On, Ln = attn(qq, kk, vv, 0.9, False)
    _close(O[0, 0, -1], On[0, 0, -1], 1e-14, "causal last row")
    # Nq > Nk causal (bottom-right aligned): the first Nq - Nk rows see nothing.
    qb = r.standard_normal((1, 1, 7, 3))
    O, L = attn(qb, kk[:, :, :4], vv[:, :, :4], 0.9, True)
    assert np.all(O[0, 0, :3] == 0.0) and np.all(np.isneginf(L[0, 0, :3])), "masked rows"
    _close(O[0, 0, 3], vv[0, 0, 0], 1e-14, "first live row sees key 0 only")
    # Key permutation (non-causal) leaves O and LSE unchanged.
    perm = r.permutation(6)
    O1, L1 = attn(q[:, :1], k[:, :1], vv, 0.7, False)
    O2, L2 = attn(q[:, :1], k[:, :1, perm], vv[:, :, perm], 0.7, False)
    _close(O2, O1, 1e-13, "permutation O")
    _close(L2, L1, 1e-13, "permutation LSE")
    # Linearity in V.
    va = r.standard_normal(k.shape)
    vb = r.standard_normal(k.shape)
    Oa, _ = attn(q, k, va, 0.7, True)
    Ob, _ = attn(q, k, vb, 0.7, True)
    Oc, _ = attn(q, k, 2.0 * va - 3.0 * vb, 0.7, True)
    _close(Oc, 2.0 * Oa - 3.0 * Ob, 1e-12, "linearity in V")


def pin_gqa_equals_mha(attn, seed=6):
    """Query head h reads KV head h // (Hq/Hkv): GQA equals MHA on K, V with
    each KV head repeated Hq/Hkv times in a row."""
    r = _rng(seed)
    B, Hq, Hkv, Nq, Nk, d = 2, 6, 2, 4, 5, 3
    q = r.standard_normal((B, Hq, Nq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    for causal in (False, True):
        O, L = attn(q, k, v, 0.6, causal)
        Om, Lm = attn(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), 0.6, causal)
        _close(O, Om, 1e-14, "GQA vs MHA O")
        _close(L, Lm, 1e-14, "GQA vs MHA LSE")


def pin_torch_sdpa(attn, seed=7):
    """Cross-check with torch's scaled_dot_product_attention on the CPU in
    float64 (the routine the pages benchmark against), with an explicit
    bottom-right causal mask; LSE against torch.logsumexp of the scaled scores."""
    import torch
    import torch.nn.functional as F

    r = _rng(seed)
    for (B, Hq, Hkv, Nq, Nk, d, causal) in [(2, 4, 2, 9, 13, 8, True), (1, 3, 3, 16, 16, 4, False),
                                            (1, 2, 1, 11, 11, 6, True)]:
        q = r.standard_normal((B, Hq, Nq, d))
        k = r.standard_normal((B, Hkv, Nk, d))
        v = r.standard_normal((B, Hkv, Nk, d))
        scale = 0.3
        O, L = attn(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        g = Hq // Hkv
        tk_r = tk.repeat_interleave(g, dim=1)
        tv_r = tv.repeat_interleave(g, dim=1)
        mask = None
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nk)[None, :]
            mask = j <= i + (Nk - Nq)
        To = F.scaled_dot_product_attention(tq, tk_r, tv_r, attn_mask=mask, scale=scale)
        s = torch.matmul(tq, tk_r.transpose(-1, -2).contiguous()) * scale
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        Tl = torch.logsumexp(s, dim=-1)
        _close(O, To.numpy(), 1e-12, "torch sdpa O")
        _close(L, Tl.numpy(), 1e-12, "torch logsumexp LSE")


ALL_PINS = [pin_brute_force, pin_identical_keys, pin_one_hot, pin_row_shift, pin_special_cases,
            pin_gqa_equals_mha, pin_torch_sdpa]
