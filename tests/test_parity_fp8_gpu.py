"""GPU parity of the fp8 forward (fa_fwd_fp8, through the C ABI) against the
fp64 oracle on the same seeded E4M3 inputs.

Tolerance, derived from the arithmetic (the task fixes none for 8-bit inputs):
the products are exact in fp32 accumulation up to ~1e-7 relative, the row sums
use the unrounded fp32 probabilities, so LSE keeps the bf16 bound (1e-3). O
differs from the exact value through the rounding of P to E4M3 before P.V:
3 mantissa bits give a relative error of at most 2^-4 for each probability in
the normal range; probabilities in the subnormal range (below 2^-6 in the
kernel's scaling, where the row's largest probability is at least 2^4) have an
absolute error of at most 2^-10, i.e. at most 2^-14 of the row's largest
probability. Hence, per element,
    |O_ij - O_ref_ij| <= 2^-4 * sum_k P_ik |V_kj|
                         + 2^-14 * max_k P_ik * sum_k |V_kj|
                         + 2^-8 |O_ref_ij| (bf16 output) + 1e-5,
with P the oracle's exact probabilities (oracle.prob_weighted_abs). Cases in
which every probability is a power of two (identical keys, one-hot selection)
have no P rounding at all and use 2^-8 |O_ref| + 1e-5."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import LSE_TOL, sample_rows, say

pytestmark = pytest.mark.gpu

DS = synth.FP8_DESCALE


def _fa():
    import exact_io_aware_17_amd as fa
    fa.lib()
    return fa


def _dev(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda")


def _run(q8, k8, v8, scale, causal, descale=DS):
    import torch
    fa = _fa()
    o, lse = fa.forward_fp8(_dev(q8), _dev(k8), _dev(v8), descale, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _inputs(w):
    return (synth.draw_e4m3(w.seed, synth.TENSOR_Q, w.q_shape), synth.draw_e4m3(w.seed, synth.TENSOR_K, w.kv_shape),
            synth.draw_e4m3(w.seed, synth.TENSOR_V, w.kv_shape))


def _bound(q, k, v, scale, causal, o_ref, q_index=None, nq=None):
    w, pmax = oracle.prob_weighted_abs(q, k, v, scale, causal, q_index=q_index, nq=nq)
    group = q.shape[1] // k.shape[1]
    vsum = np.repeat(np.abs(v).sum(axis=2), group, axis=1)  # [B, Hq, d], all keys
    return 2.0 ** -4 * w + 2.0 ** -14 * pmax[..., None] * vsum[:, :, None, :] + 2.0 ** -8 * np.abs(o_ref) + 1e-5


def _check(o, lse, o_ref, lse_ref, bound, what):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: rows without keys differ"
    assert not np.isnan(o).any() and not np.isnan(lse).any(), f"{what}: NaN"
    fin = np.isfinite(lse_ref)
    e_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    ratio = np.abs(o - o_ref) / bound
    say(f"  {what}: max|dO| = {np.max(np.abs(o - o_ref)):.3e}, max |dO|/bound = {ratio.max():.3f}, "
        f"mean |dO|/bound = {ratio.mean():.4f}, max|dLSE| = {e_l:.3e}")
    assert ratio.max() <= 1.0, f"{what}: O outside the E4M3 rounding bound (ratio {ratio.max():.3f})"
    assert e_l <= LSE_TOL, f"{what}: max|LSE-LSE_ref| = {e_l:.3e}"


SMALL = [
    synth.Workload("fp8_single_head_n256", 1, 1, 1, 256, 256, 128),
    synth.Workload("fp8_ragged_gqa", 2, 4, 2, 200, 333, 128, seed=1),
    synth.Workload("fp8_ragged_gqa_causal", 2, 4, 2, 200, 333, 128, causal=True, seed=2),
    synth.Workload("fp8_more_queries_than_keys_causal", 1, 3, 1, 300, 70, 128, causal=True, seed=5),
    synth.Workload("fp8_one_query_one_key", 1, 1, 1, 1, 1, 128),
    synth.Workload("fp8_keys_below_one_tile", 1, 2, 2, 300, 17, 128, seed=4),
    synth.Workload("fp8_square_causal_3_tiles", 1, 2, 2, 384, 384, 128, causal=True),
    synth.Workload("fp8_one_query", 2, 8, 2, 1, 1000, 128, seed=8),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fp8_full_oracle(w):
    say(f"case fp8 full {w.name}")
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, w.causal)
    q, k, v = (oracle.e4m3_decode(t) * DS[i] for i, t in enumerate((q8, k8, v8)))
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    o_ref2, lse_ref2 = oracle.attention_fp8(q8, k8, v8, DS, w.scale, w.causal)
    assert np.array_equal(o_ref, o_ref2) and np.array_equal(lse_ref, lse_ref2)
    _check(o, lse, o_ref, lse_ref, _bound(q, k, v, w.scale, w.causal, o_ref), w.name)


def _random_shapes(n=16, seed=2028):
    """Seeded mixed shapes at d = 128: batch 1-2, 1-3 KV heads, GQA 1/2/4,
    1..399 rows and keys, with and without causal."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.integers(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append(synth.Workload(f"fp8_random_{i}", int(rng.integers(1, 3)), hq, hkv, int(rng.integers(1, 400)),
                                  int(rng.integers(1, 400)), 128, causal=bool(rng.integers(0, 2)), seed=400 + i))
    return out


@pytest.mark.parametrize("w", _random_shapes(), ids=lambda w: w.name)
def test_fp8_random_shapes(w):
    say(f"case fp8 random {w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} {w.Nq}x{w.Nk} causal={w.causal}")
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, w.causal)
    q, k, v = (oracle.e4m3_decode(t) * DS[i] for i, t in enumerate((q8, k8, v8)))
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    _check(o, lse, o_ref, lse_ref, _bound(q, k, v, w.scale, w.causal, o_ref), w.name)


def test_fp8_pages_shape_full_size_sampled():
    """The benchmark's launch (the pages' shape, B1 H8 4096x8192, E4M3), with
    the oracle computing sampled rows of three heads."""
    w = synth.WORKLOADS["pages_shape_fp8_h8_q4096_kv8192"]
    say(f"case fp8 full-size {w.name}")
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, w.causal)
    rows = sample_rows(w.Nq)
    for h in (0, 3, 7):
        q = oracle.e4m3_decode(q8[:, h:h + 1, rows]) * DS[0]
        k = oracle.e4m3_decode(k8[:, h:h + 1]) * DS[1]
        v = oracle.e4m3_decode(v8[:, h:h + 1]) * DS[2]
        o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal, q_index=rows, nq=w.Nq)
        bound = _bound(q, k, v, w.scale, w.causal, o_ref, q_index=rows, nq=w.Nq)
        _check(o[:, h:h + 1, rows], lse[:, h:h + 1, rows], o_ref, lse_ref, bound, f"{w.name} head {h}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_large_shapes_sampled(causal):
    """The largest fp8 launches: B4 H16 2048^2 and, causal, B1 H32 16384^2;
    sampled rows of two heads against the oracle."""
    w = (synth.Workload("fp8_long_causal_h32_n16384", 1, 32, 32, 16384, 16384, 128, causal=True) if causal
         else synth.Workload("fp8_batched_b4h16_n2048", 4, 16, 16, 2048, 2048, 128))
    say(f"case fp8 full-size {w.name}")
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, w.causal)
    rows = sample_rows(w.Nq)
    for (b, h) in ((0, 0), (w.B - 1, w.Hq - 1)):
        q = oracle.e4m3_decode(q8[b:b + 1, h:h + 1, rows]) * DS[0]
        k = oracle.e4m3_decode(k8[b:b + 1, h:h + 1]) * DS[1]
        v = oracle.e4m3_decode(v8[b:b + 1, h:h + 1]) * DS[2]
        o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal, q_index=rows, nq=w.Nq)
        bound = _bound(q, k, v, w.scale, w.causal, o_ref, q_index=rows, nq=w.Nq)
        _check(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], o_ref, lse_ref, bound, f"{w.name} ({b},{h})")


def test_fp8_identical_keys_exact_probabilities():
    """Every key equal: every probability is the same power of two, so P is
    exact in E4M3 and O is the column mean of V (bf16 output rounding only);
    LSE = s + ln Nk."""
    r = np.random.default_rng(11)
    Nq, Nk, d = 130, 200, 128
    q8 = synth.e4m3_bits(r.standard_normal((1, 2, Nq, d)) / DS[0])
    krow = synth.e4m3_bits(r.standard_normal(d) / DS[1])
    k8 = np.broadcast_to(krow, (1, 1, Nk, d)).copy()
    v8 = synth.e4m3_bits(r.standard_normal((1, 1, Nk, d)) / DS[2])
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(q8, k8, v8, scale, False)
    o_ref, lse_ref = oracle.attention_fp8(q8, k8, v8, DS, scale, False)
    assert np.max(np.abs(o - o_ref) - (2.0 ** -8 * np.abs(o_ref) + 1e-5)) <= 0
    assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL


def test_fp8_one_hot_selection():
    """Key j is c*e_j, query i is e_t(i) (E4M3 exact values): the logit of the
    chosen key is ~45 above the others, its probability rounds to exactly the
    largest power of two and the rest underflow, so O_i is V_t(i)."""
    d, Nk, Nq = 128, 128, 96
    q = np.zeros((1, 1, Nq, d))
    t = (np.arange(Nq) * 37) % Nk
    q[0, 0, np.arange(Nq), t] = 1.0
    k = np.zeros((1, 1, Nk, d))
    k[0, 0, np.arange(Nk), np.arange(Nk)] = 448.0
    q8 = synth.e4m3_bits(q)
    k8 = synth.e4m3_bits(k)
    v8 = synth.e4m3_bits(np.random.default_rng(12).standard_normal((1, 1, Nk, d)) / DS[2])
    descale = (1.0, 1.0, DS[2])
    scale = 0.1  # logit 44.8 for the chosen key, 0 for the others
    o, lse = _run(q8, k8, v8, scale, False, descale=descale)
    o_ref, lse_ref = oracle.attention_fp8(q8, k8, v8, descale, scale, False)
    vsel = oracle.e4m3_decode(v8[0, 0, t]) * DS[2]
    assert np.max(np.abs(o[0, 0] - vsel) - (2.0 ** -8 * np.abs(vsel) + 1e-5)) <= 0
    assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL


def test_fp8_descales_fold_into_score_scale():
    """Only the product q_descale * k_descale enters the scores: (2a, b/2, c)
    gives bitwise the same output as (a, b, c)."""
    w = synth.Workload("fp8_descale", 1, 2, 1, 150, 260, 128, causal=True, seed=9)
    q8, k8, v8 = _inputs(w)
    o1, l1 = _run(q8, k8, v8, w.scale, True, descale=DS)
    o2, l2 = _run(q8, k8, v8, w.scale, True, descale=(DS[0] * 2, DS[1] / 2, DS[2]))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8_deterministic_and_float8_dtype():
    import torch
    fa = _fa()
    w = synth.Workload("fp8_det", 1, 4, 2, 300, 500, 128, seed=10)
    q8, k8, v8 = (_dev(x) for x in _inputs(w))
    o1, l1 = fa.forward_fp8(q8, k8, v8, DS, scale=w.scale)
    o2, l2 = fa.forward_fp8(q8.view(torch.float8_e4m3fn), k8.view(torch.float8_e4m3fn),
                            v8.view(torch.float8_e4m3fn), DS, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_argument_errors():
    import torch
    fa = _fa()
    q = torch.zeros((1, 2, 8, 64), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8(q, q, q, o, lse, DS)
    assert e.value.status == 3  # head size 64: unsupported
    q = torch.zeros((1, 2, 8, 128), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
    for bad in [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("inf")), (1e-30, 1e-30, 1.0)]:
        with pytest.raises(fa.FaError) as e:
            fa.fa_fwd_fp8(q, q, q, o, lse, bad)
        assert e.value.status == 7
    with pytest.raises(TypeError):
        fa.fa_fwd_fp8(q.to(torch.bfloat16), q, q, o, lse, DS)
    # Empty batch: nothing to do.
    z = torch.zeros((0, 2, 8, 128), dtype=torch.uint8, device="cuda")
    fa.fa_fwd_fp8(z, z, z, torch.empty((0, 2, 8, 128), dtype=torch.bfloat16, device="cuda"),
                  torch.empty((0, 2, 8), dtype=torch.float32, device="cuda"), DS)


def test_fp8_no_keys_and_no_queries():
    """Nk = 0: every row has no key (O = 0, LSE = -inf); Nq = 0: nothing to do."""
    w = synth.Workload("fp8_no_keys", 1, 2, 1, 40, 0, 128)
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, False)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    w = synth.Workload("fp8_no_queries", 1, 2, 1, 0, 40, 128)
    q8, k8, v8 = _inputs(w)
    o, lse = _run(q8, k8, v8, w.scale, False)
    assert o.size == 0 and lse.size == 0
