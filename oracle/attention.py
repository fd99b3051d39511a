"""Plain, slow, fp64 definition of exact attention and of its split-KV form.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

Sources (web pages; cited by title and section):

* "flash attention v3 paper" search-result page, the standard self-attention
  snippet: for per-head matrices Q, K, V of shape (N, d), S = Q K^T, P is the
  row-wise softmax of S, O = P V (the snippet leaves out the scale and the mask).
* "Flash Attention on the 5090 in CUDA C++" (Hacker News digest), the
  "Flash Attention 2 algorithm" pseudocode: scale = DIM^-0.5 multiplies the
  product Q_tile K_tile^T; an O tile is zeroed, KV tiles are visited in order,
  an online softmax runs over each score tile, O accumulates (scores) @ V_tile,
  and O is stored once.
* Same page, "v1 -- basic version", online-softmax bullets: the running max m,
  the running denominator d (called ``l`` here, to keep d for the head size),
  and the rescale of the earlier partial O by exp(m_prev - m) (together with
  d_prev / d in the normalised form).
* "Flash Attention" (aiunderstanding.org), deep dive and FAQ: the method is
  exact (same result as the plain computation); tiles plus the online softmax
  avoid storing the N x N matrix.

Readings where the pages are silent (each also listed in the design notes):

* Layout [B, H, N, d], d innermost; LSE is [B, Hq, Nq].
* GQA: query head h reads KV head h // (Hq // Hkv).
* Causal mask, bottom-right aligned: key j is visible to query i iff
  j <= i + (Nk - Nq).  For Nq == Nk this is the lower-triangular mask.
* LSE_i = m_i + ln(l_i): natural log of the sum of exp of the *scaled* scores.
* A row with no visible key has O = 0 and LSE = -inf; a split chunk with no
  key gets the same partial result and weight zero in the combine.
* Split chunks are contiguous along keys: chunk s covers
  [s*C, min(Nk, (s+1)*C)) with C = ceil(Nk / num_splits).
* Paged K/V (PagedAttention is only named on the "flash attention v3 paper"
  search-result page): a cache [num_pages, Hkv, page, d] whose page p holds
  `page` consecutive keys of each KV head, a table [B, max_pages] naming the
  physical page of each logical page of a sequence, and one key count per
  sequence. Paged attention is plain attention over the gathered keys.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, _, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nk, d


def _rows(qh, kh, vh, scale, last_visible, key_lo):
    """Two-pass softmax attention for a block of query rows over keys
    [key_lo, key_lo + len(kh)).  ``last_visible[r]`` is the largest global key
    index row r may see (None: all keys).  Returns (O rows, LSE rows)."""
    # Scores: (Q K^T) * scale, fully materialised, scale applied after the
    # product as in the pseudocode.
    s = (qh @ kh.T) * scale
    if last_visible is not None:
        keys = key_lo + np.arange(kh.shape[0])
        s[keys[None, :] > last_visible[:, None]] = NEG_INF
    # Pass 1: row max.
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    alive = np.isfinite(m)
    m_safe = np.where(alive, m, 0.0)
    # Pass 2: exponentials, row sum, normalised probabilities.
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[alive] = e[alive] / l[alive, None]
    o = p @ vh
    lse = np.full(s.shape[0], NEG_INF)
    lse[alive] = m[alive] + np.log(l[alive])
    o[~alive] = 0.0
    return o, lse


def attention(q, k, v, scale, causal=False, q_index=None, nq=None, key_range=None, row_block=2048):
    """Exact attention, O = softmax(Q K^T * scale) V, with LSE.

    q: [B, Hq, n, d] float64 (n query rows; by default all Nq rows).
    k, v: [B, Hkv, Nk, d] float64.
    q_index: global query index of each of the n rows (default 0..n-1).
    nq: total number of queries Nq (needed by the causal alignment; default n).
    key_range: (lo, hi) to restrict attention to keys [lo, hi) (split chunks).
    Rows are independent, so they are processed in blocks of ``row_block`` to
    bound memory; each block is still the materialised two-pass definition.
    Returns (O [B, Hq, n, d], LSE [B, Hq, n]) in float64.
    """
    B, Hq, Hkv, Nk, d = _check(q, k, v)
    n = q.shape[2]
    group = Hq // Hkv
    q_index = np.arange(n) if q_index is None else np.asarray(q_index)
    nq = n if nq is None else nq
    lo, hi = (0, Nk) if key_range is None else key_range
    o = np.zeros((B, Hq, n, d))
    lse = np.full((B, Hq, n), NEG_INF)
    if hi <= lo:
        return o, lse
    for b in range(B):
        for h in range(Hq):
            g = h // group
            kh = k[b, g, lo:hi]
            vh = v[b, g, lo:hi]
            for r0 in range(0, n, row_block):
                r1 = min(n, r0 + row_block)
                last = (q_index[r0:r1] + (Nk - nq)) if causal else None
                o[b, h, r0:r1], lse[b, h, r0:r1] = _rows(q[b, h, r0:r1], kh, vh, scale, last, lo)
    return o, lse


def attention_online(q, k, v, scale, causal=False, tile=64, form="fa2"):
    """The tiled online-softmax recurrence, in fp64, used only to check that the
    recurrence reaches the same result as :func:`attention`.

    Follows the pseudocode's loop (zero O, visit KV tiles in order, score tile,
    online softmax, accumulate into O, store once).  ``form="fa1"`` keeps O
    normalised after every tile, as in the v1 bullets:
        m = max(m_prev, rowmax S_t)
        l = l_prev * exp(m_prev - m) + sum exp(S_t - m)
        O = O_prev * (l_prev / l) * exp(m_prev - m) + (exp(S_t - m) / l) @ V_t
    ``form="fa2"`` keeps O unnormalised and divides by l once at the end.
    """
    if form not in ("fa1", "fa2"):
        raise ValueError(form)
    B, Hq, Hkv, Nk, d = _check(q, k, v)
    Nq = q.shape[2]
    group = Hq // Hkv
    o_all = np.zeros((B, Hq, Nq, d))
    lse_all = np.full((B, Hq, Nq), NEG_INF)
    last = np.arange(Nq) + (Nk - Nq)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh = q[b, h]
            m = np.full(Nq, NEG_INF)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, d))
            for j0 in range(0, Nk, tile):
                j1 = min(Nk, j0 + tile)
                s = (qh @ k[b, g, j0:j1].T) * scale
                if causal:
                    s[np.arange(j0, j1)[None, :] > last[:, None]] = NEG_INF
                m_tile = s.max(axis=1)
                m_new = np.maximum(m, m_tile)
                live = np.isfinite(m_new)
                base = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(np.where(np.isfinite(m), m, -np.inf) - base), 1.0)
                e = np.exp(s - base[:, None])
                l_new = l * alpha + e.sum(axis=1)
                if form == "fa1":
                    ratio = np.zeros(Nq)
                    inv = np.zeros(Nq)
                    nz = l_new > 0
                    ratio[nz] = l[nz] / l_new[nz] * alpha[nz]
                    inv[nz] = 1.0 / l_new[nz]
                    acc = acc * ratio[:, None] + (e * inv[:, None]) @ v[b, g, j0:j1]
                else:
                    acc = acc * alpha[:, None] + e @ v[b, g, j0:j1]
                m, l = m_new, l_new
            live = l > 0
            if form == "fa2":
                acc[live] /= l[live, None]
            acc[~live] = 0.0
            o_all[b, h] = acc
            lse_all[b, h, live] = m[live] + np.log(l[live])
    return o_all, lse_all


def split_bounds(nk, num_splits):
    """Contiguous key chunks: chunk s is [s*C, min(nk, (s+1)*C)), C = ceil(nk/num_splits)."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    c = -(-nk // num_splits)
    return [(min(nk, s * c), min(nk, (s + 1) * c)) for s in range(num_splits)]


def splitkv_partials(q, k, v, scale, num_splits, causal=False):
    """Per-chunk attention: for every chunk, the exact attention of each query
    row over that chunk's keys alone (normalised O_s and its LSE_s).

    Returns (O_part [B, Hq, S, Nq, d], LSE_part [B, Hq, S, Nq]).
    """
    B, Hq, Hkv, Nk, d = _check(q, k, v)
    Nq = q.shape[2]
    bounds = split_bounds(Nk, num_splits)
    o_part = np.zeros((B, Hq, num_splits, Nq, d))
    lse_part = np.full((B, Hq, num_splits, Nq), NEG_INF)
    for s, (lo, hi) in enumerate(bounds):
        o_part[:, :, s], lse_part[:, :, s] = attention(q, k, v, scale, causal, key_range=(lo, hi))
    return o_part, lse_part


def combine(o_part, lse_part):
    """LSE-weighted merge of chunk results, the whole-chunk form of the online
    rescale: with M = max_s LSE_s and w_s = exp(LSE_s - M),
    O = sum_s w_s O_s / sum_s w_s and LSE = M + ln(sum_s w_s).
    Chunks with LSE_s = -inf get weight zero; if every chunk is empty the row
    is O = 0, LSE = -inf.
    o_part: [..., S, n, d]; lse_part: [..., S, n].  Returns (O [..., n, d], LSE [..., n]).
    """
    lse_part = np.asarray(lse_part, dtype=np.float64)
    o_part = np.asarray(o_part, dtype=np.float64)
    m = lse_part.max(axis=-2)
    alive = np.isfinite(m)
    m_safe = np.where(alive, m, 0.0)
    w = np.exp(lse_part - m_safe[..., None, :])
    den = w.sum(axis=-2)
    num = (w[..., None] * o_part).sum(axis=-3)
    o = np.zeros_like(num)
    o[alive] = num[alive] / den[alive][..., None]
    lse = np.full(m.shape, NEG_INF)
    lse[alive] = m[alive] + np.log(den[alive])
    return o, lse



def paged_gather(k_cache, v_cache, block_table, seq_len, b):
    """Keys 0 .. seq_len-1 of sequence b, gathered page by page from the
    caches [num_pages, Hkv, page, d]: logical page j is physical page
    block_table[b, j].  Returns (k [Hkv, seq_len, d], v [Hkv, seq_len, d])."""
    num_pages, Hkv, page, d = k_cache.shape
    n_pages = -(-seq_len // page)
    pages = np.asarray(block_table[b, :n_pages], dtype=np.int64)
    k = np.concatenate([k_cache[p] for p in pages], axis=1) if n_pages else np.zeros((Hkv, 0, d))
    v = np.concatenate([v_cache[p] for p in pages], axis=1) if n_pages else np.zeros((Hkv, 0, d))
    return k[:, :seq_len], v[:, :seq_len]


def paged_attention(q, k_cache, v_cache, block_table, seq_lens, scale, causal=False):
    """Attention of sequence b over its own seq_lens[b] keys, gathered from the
    page caches; each sequence is the plain definition with Nk = seq_lens[b]
    (so the causal diagonal sits at seq_lens[b] - Nq).
    q [B, Hq, Nq, d]; returns (O [B, Hq, Nq, d], LSE [B, Hq, Nq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), NEG_INF)
    for b in range(B):
        k, v = paged_gather(k_cache, v_cache, block_table, int(seq_lens[b]), b)
        ob, lb = attention(q[b:b + 1], k[None], v[None], scale, causal)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse
