"""The oracle against its pins (CPU only).

The pins are facts the pages and mathematics fix (brute force, closed forms,
invariants, a library cross-check).  The mutation tests apply the same pins to
plausible wrong variants of the oracle and require each to be caught.
"""
import functools

import numpy as np
import pytest

import oracle
import oracle_pins as P


def _oracle(q, k, v, scale, causal):
    return oracle.attention(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pins(pin):
    pin(_oracle)


@pytest.mark.parametrize("form", ["fa1", "fa2"])
@pytest.mark.parametrize("tile", [1, 3, 7, 64, 1000])
def test_online_recurrence_pins(form, tile):
    """The tiled online-softmax recurrence (both forms) meets every pin."""
    fn = functools.partial(_online, form=form, tile=tile)
    for pin in P.ALL_PINS:
        pin(fn)


def _online(q, k, v, scale, causal, form, tile):
    return oracle.attention_online(q, k, v, scale, causal, tile=tile, form=form)


@pytest.mark.parametrize("form", ["fa1", "fa2"])
@pytest.mark.parametrize("tile", [1, 7, 64, 200])
def test_online_equals_two_pass(form, tile):
    r = np.random.default_rng(11)
    for causal in (False, True):
        q = r.standard_normal((2, 4, 37, 16))
        k = r.standard_normal((2, 2, 45, 16))
        v = r.standard_normal((2, 2, 45, 16))
        O, L = oracle.attention(q, k, v, 0.25, causal)
        O2, L2 = oracle.attention_online(q, k, v, 0.25, causal, tile=tile, form=form)
        np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L2, L, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 5, 16, 45, 60])
def test_split_combine_equals_unsplit(splits):
    """Combining per-chunk (O_s, LSE_s) reproduces unsplit attention for dividing,
    non-dividing and over-long split counts (the last: empty chunks)."""
    r = np.random.default_rng(12)
    for causal in (False, True):
        q = r.standard_normal((2, 4, 3, 8))
        k = r.standard_normal((2, 2, 45, 8))
        v = r.standard_normal((2, 2, 45, 8))
        O, L = oracle.attention(q, k, v, 0.4, causal)
        op, lp = oracle.splitkv_partials(q, k, v, 0.4, splits, causal)
        assert op.shape == (2, 4, splits, 3, 8) and lp.shape == (2, 4, splits, 3)
        Oc, Lc = oracle.combine(op, lp)
        np.testing.assert_allclose(Oc, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lc, L, rtol=1e-13, atol=1e-12)


def test_split_single_chunk_is_identity():
    r = np.random.default_rng(13)
    q = r.standard_normal((1, 2, 1, 8))
    k = r.standard_normal((1, 1, 30, 8))
    v = r.standard_normal((1, 1, 30, 8))
    op, lp = oracle.splitkv_partials(q, k, v, 0.4, 1)
    O, L = oracle.attention(q, k, v, 0.4)
    np.testing.assert_array_equal(op[:, :, 0], O)
    np.testing.assert_array_equal(lp[:, :, 0], L)
    Oc, Lc = oracle.combine(op, lp)
    np.testing.assert_allclose(Oc, O, atol=1e-15, rtol=0)


def test_split_bounds():
    assert oracle.split_bounds(8192, 16) == [(512 * s, 512 * (s + 1)) for s in range(16)]
    assert oracle.split_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.split_bounds(3, 5) == [(0, 1), (1, 2), (2, 3), (3, 3), (3, 3)]


def test_empty_chunks_have_zero_weight():
    op = np.zeros((1, 1, 3, 2, 4))
    lp = np.full((1, 1, 3, 2), -np.inf)
    op[0, 0, 1] = 7.0
    lp[0, 0, 1] = 0.5
    O, L = oracle.combine(op, lp)
    np.testing.assert_array_equal(O[0, 0], np.full((2, 4), 7.0))
    np.testing.assert_array_equal(L[0, 0], [0.5, 0.5])
    O, L = oracle.combine(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_sampled_rows_equal_full():
    """Row-sampled calls (used for large workloads) give the same rows."""
    r = np.random.default_rng(14)
    q = r.standard_normal((1, 2, 50, 8))
    k = r.standard_normal((1, 1, 64, 8))
    v = r.standard_normal((1, 1, 64, 8))
    O, L = oracle.attention(q, k, v, 0.3, True)
    rows = np.array([0, 3, 17, 49])
    Os, Ls = oracle.attention(q[:, :, rows], k, v, 0.3, True, q_index=rows, nq=50)
    np.testing.assert_array_equal(Os, O[:, :, rows])
    np.testing.assert_array_equal(Ls, L[:, :, rows])
    Ob, Lb = oracle.attention(q, k, v, 0.3, True, row_block=7)
    np.testing.assert_allclose(Ob, O, atol=1e-15, rtol=0)


# ---------------------------------------------------------------------------
# Mutation tests: plausible mistakes, each of which some pin must reject.

def _generic(q, k, v, scale, causal, *, scale_fn=lambda s: s, mask_fn=None, group_fn=None,
             lse_fn=None, shift=True, use_v=True, axis=1, keys_fn=None):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Nq, d))
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = group_fn(h, G, Hkv) if group_fn else h // G
            kk = k[b, g]
            vv = v[b, g] if use_v else k[b, g]
            if keys_fn:
                kk, vv = keys_fn(kk), keys_fn(vv)
            s = (q[b, h] @ kk.T) * scale_fn(scale)
            if causal:
                i = np.arange(Nq)[:, None]
                j = np.arange(kk.shape[0])[None, :]
                bad = mask_fn(i, j, Nq, Nk) if mask_fn else j > i + (Nk - Nq)
                s = np.where(bad, -np.inf, s)
            with np.errstate(all="ignore"):
                m = s.max(axis=axis, keepdims=True) if shift else np.zeros((1, 1))
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(s - m)
                l = e.sum(axis=axis, keepdims=True)
                p = e / l
                O[b, h] = np.nan_to_num(p @ vv) if axis == 1 else (p @ vv)
                lse = (m + np.log(l)).reshape(-1) if axis == 1 else np.log(np.exp(s).sum(1))
                L[b, h] = lse_fn(lse, m.reshape(-1), l.reshape(-1)) if lse_fn else lse
    return O, L


MUTANTS = {
    "scale dropped": dict(scale_fn=lambda s: 1.0),
    "scale squared": dict(scale_fn=lambda s: s * s),
    "causal top-left aligned": dict(mask_fn=lambda i, j, nq, nk: j > i),
    "causal mask strict": dict(mask_fn=lambda i, j, nq, nk: j >= i + (nk - nq)),
    "GQA interleaved heads": dict(group_fn=lambda h, G, Hkv: h % Hkv),
    "LSE in log2": dict(lse_fn=lambda lse, m, l: m + np.log2(l)),
    "LSE without max": dict(lse_fn=lambda lse, m, l: np.log(l)),
    "no max subtraction": dict(shift=False),
    "K used as V": dict(use_v=False),
    "softmax over the query axis": dict(axis=0),
    "last key dropped": dict(keys_fn=lambda x: x[:-1]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    fn = functools.partial(_generic, **MUTANTS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant '{name}'"


def test_generic_unmutated_passes():
    """The harness used for the mutants is itself correct when unmutated."""
    for pin in P.ALL_PINS:
        pin(_generic)


# --- paged K/V -------------------------------------------------------------

def _paged_cache(k, v, page, seed, spare=3):
    """A page cache [num_pages, Hkv, page, d] holding contiguous K/V
    [B, Hkv, Nk, d] under a random page permutation (plus unused pages full of
    noise), and its block table [B, max_pages]."""
    r = np.random.default_rng(seed)
    B, Hkv, Nk, d = k.shape
    max_pages = -(-Nk // page)
    num_pages = B * max_pages + spare
    perm = r.permutation(num_pages)
    kc = r.standard_normal((num_pages, Hkv, page, d))
    vc = r.standard_normal((num_pages, Hkv, page, d))
    table = np.zeros((B, max_pages), dtype=np.int32)
    for b in range(B):
        for j in range(max_pages):
            p = perm[b * max_pages + j]
            table[b, j] = p
            n = min(page, Nk - j * page)
            kc[p, :, :n] = k[b, :, j * page: j * page + n]
            vc[p, :, :n] = v[b, :, j * page: j * page + n]
    return kc, vc, table


@pytest.mark.parametrize("page", [1, 4, 16])
def test_paged_gather_gives_back_the_keys(page):
    r = np.random.default_rng(11)
    k = r.standard_normal((3, 2, 37, 4))
    v = r.standard_normal((3, 2, 37, 4))
    kc, vc, table = _paged_cache(k, v, page, seed=page)
    for b, L in ((0, 37), (1, 20), (2, 0), (2, 1)):
        kg, vg = oracle.paged_gather(kc, vc, table, L, b)
        assert kg.shape == (2, L, 4) and vg.shape == (2, L, 4)
        assert np.array_equal(kg, k[b, :, :L]) and np.array_equal(vg, v[b, :, :L])


@pytest.mark.parametrize("causal", [False, True])
def test_paged_attention_is_attention_over_each_sequence(causal):
    r = np.random.default_rng(12)
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 3, 50, 8
    q = r.standard_normal((B, Hq, Nq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    kc, vc, table = _paged_cache(k, v, 16, seed=3)
    lens = np.array([50, 17, 2], dtype=np.int32)
    o, lse = oracle.paged_attention(q, kc, vc, table, lens, 0.3, causal)
    for b in range(B):
        L = int(lens[b])
        ob, lb = oracle.attention(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.3, causal)
        assert np.allclose(o[b], ob[0], rtol=0, atol=1e-13) and np.allclose(lse[b], lb[0], rtol=0, atol=1e-13)
    # rows whose causal window holds no key: O = 0, LSE = -inf
    if causal:
        assert np.all(np.isneginf(lse[2, :, 0])) and np.all(o[2, :, 0] == 0)


def test_paged_attention_brute_force():
    """A tiny paged case against pure-Python loops on the gathered keys."""
    r = np.random.default_rng(13)
    k = r.standard_normal((2, 1, 5, 3))
    v = r.standard_normal((2, 1, 5, 3))
    q = r.standard_normal((2, 2, 2, 3))
    kc, vc, table = _paged_cache(k, v, 2, seed=4)
    lens = np.array([5, 3], dtype=np.int32)
    for causal in (False, True):
        o, lse = oracle.paged_attention(q, kc, vc, table, lens, 0.7, causal)
        for b in range(2):
            L = int(lens[b])
            ob, lb = P.brute_attention(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.7, causal)
            assert np.allclose(o[b], ob[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[b], lb[0], rtol=0, atol=1e-12)
