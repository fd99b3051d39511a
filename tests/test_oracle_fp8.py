"""Pins of the fp8 side of the oracle (CPU only): the OCP E4M3 decoder, the
descale reading of attention over fp8 inputs, and the probability weights
used to bound the rounding of P.  Also the seeded E4M3 input encoder."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_e4m3_closed_form_codes():
    # Values fixed by the format: bias 7, 3 mantissa bits, subnormals, no inf.
    cases = {
        0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x30: 0.5, 0x7E: 448.0,
        0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x77: 240.0,
        0xC0: -2.0, 0xFE: -448.0, 0x58: 16.0,
    }
    for code, val in cases.items():
        assert oracle.e4m3_value(code) == val, hex(code)
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0 and oracle.e4m3_value(0x80) == 0.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_decode_matches_library_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_e4m3_positive_codes_are_increasing():
    v = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0) and v[-1] == 448.0 and len(v) == 127


def test_e4m3_encoder_rounds_to_nearest_even():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(100000) * 60, r.uniform(-2 ** -5, 2 ** -5, 20000),
                        [0.0, 448.0, 1.0625, 17.0, 2.0 ** -10, 3 * 2.0 ** -10, 460.0, 1e6]])
    codes = synth.e4m3_bits(x)
    vals = oracle.e4m3_decode(codes)
    grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), 448.0)
    # Nearest finite value; on a tie the one with an even code.
    idx = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo, hi = grid[idx - 1], grid[idx]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (idx % 2 == 0))
    want = np.where(pick_hi, hi, lo) * np.where(np.signbit(x), -1.0, 1.0)
    assert np.array_equal(vals, want)
    assert not np.any((codes & 0x7F) == 0x7F)


def _small(seed=0, B=1, Hq=2, Hkv=1, Nq=9, Nk=13, d=8):
    r = np.random.default_rng(seed)
    q8 = synth.e4m3_bits(r.standard_normal((B, Hq, Nq, d)) / synth.FP8_DESCALE[0])
    k8 = synth.e4m3_bits(r.standard_normal((B, Hkv, Nk, d)) / synth.FP8_DESCALE[1])
    v8 = synth.e4m3_bits(r.standard_normal((B, Hkv, Nk, d)) / synth.FP8_DESCALE[2])
    return q8, k8, v8


@pytest.mark.parametrize("causal", [False, True])
def test_descales_act_on_scores_and_output(causal):
    """Q and K descales multiply every score (so they fold into the score
    scale); the V descale multiplies O and leaves LSE alone."""
    q8, k8, v8 = _small()
    ds = (0.03, 0.02, 0.05)
    scale = 0.3
    o, lse = oracle.attention_fp8(q8, k8, v8, ds, scale, causal)
    q, k, v = (oracle.e4m3_decode(t) for t in (q8, k8, v8))
    o2, lse2 = oracle.attention(q, k, v, scale * ds[0] * ds[1], causal)
    np.testing.assert_allclose(o, o2 * ds[2], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-13)


def test_prob_weighted_abs_closed_forms():
    r = np.random.default_rng(5)
    B, H, Nq, Nk, d = 1, 2, 5, 11, 6
    q = r.standard_normal((B, H, Nq, d))
    k = r.standard_normal((B, H, Nk, d))
    # V = 1: sum_j P_ij |V_j| = 1 for every row.
    w, pmax = oracle.prob_weighted_abs(q, k, np.ones((B, H, Nk, d)), 0.5)
    np.testing.assert_allclose(w, 1.0, rtol=1e-13)
    # Identical keys: P is uniform, Pmax = 1 / Nk, W = column mean of |V|.
    v = r.standard_normal((B, H, Nk, d))
    k_same = np.broadcast_to(k[:, :, :1], k.shape).copy()
    w, pmax = oracle.prob_weighted_abs(q, k_same, v, 0.5)
    np.testing.assert_allclose(pmax, 1.0 / Nk, rtol=1e-13)
    np.testing.assert_allclose(w, np.broadcast_to(np.abs(v).mean(axis=2, keepdims=True), w.shape), rtol=1e-12)
    # One-hot selection (logit 45): Pmax ~ 1, W = |selected V row|.
    kk = np.zeros((1, 1, d, d))
    kk[0, 0] = np.eye(d) * 90.0
    qq = np.zeros((1, 1, d, d))
    qq[0, 0] = np.eye(d)[::-1]
    vv = r.standard_normal((1, 1, d, d))
    w, pmax = oracle.prob_weighted_abs(qq, kk, vv, 0.5)
    np.testing.assert_allclose(pmax, 1.0, rtol=1e-15, atol=1e-18)
    np.testing.assert_allclose(w[0, 0], np.abs(vv[0, 0, ::-1]), rtol=1e-15, atol=1e-17)


def test_prob_weighted_abs_brute_force_causal():
    r = np.random.default_rng(6)
    Nq, Nk, d = 4, 6, 3
    q = r.standard_normal((1, 2, Nq, d))
    k = r.standard_normal((1, 1, Nk, d))
    v = r.standard_normal((1, 1, Nk, d))
    w, pmax = oracle.prob_weighted_abs(q, k, v, 0.7, causal=True)
    for h in range(2):
        for i in range(Nq):
            keys = [j for j in range(Nk) if j <= i + (Nk - Nq)]
            s = [0.7 * math.fsum(q[0, h, i, t] * k[0, 0, j, t] for t in range(d)) for j in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = math.fsum(e)
            p = [x / tot for x in e]
            assert abs(pmax[0, h, i] - max(p)) < 1e-14
            for t in range(d):
                ref = math.fsum(p[n] * abs(v[0, 0, j, t]) for n, j in enumerate(keys))
                assert abs(w[0, h, i, t] - ref) < 1e-14


def test_draw_e4m3_is_the_encoded_draw():
    shape = (1, 2, 33, 16)
    codes = synth.draw_e4m3(0, synth.TENSOR_K, shape)
    raw = synth.draw(0, synth.TENSOR_K, shape).astype(np.float64) / synth.FP8_DESCALE[synth.TENSOR_K]
    assert codes.dtype == np.uint8 and codes.shape == shape
    assert np.array_equal(codes, synth.e4m3_bits(raw))
    # Only one head drawn: the same bytes as in the full draw.
    one = synth.draw_e4m3(0, synth.TENSOR_K, shape, heads=[(0, 1)])
    assert np.array_equal(one[0], codes[0, 1])
