"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 oracle (oracle.attention_backward) on the same seeded bf16 inputs.

Tolerance, derived from the arithmetic (the task fixes none for gradients),
per element, from the exact quantities of the oracle (P, dP = dO V^T,
D = rowsum(dO o O), dS = P (dP - D)) and the operand magnitudes:
  * P carries a relative error of about 2^-16 scale sum_c |Q_ic||K_jc| (the
    fp32 score) plus 2^-17 (the fp32 LSE of the forward, exp2): relP_ij;
  * dP and D are fp32 sums of d exact bf16 products (at most 2 d 2^-24 of the
    sum of |terms|: A_ij = sum_c |dO_ic||V_jc|, E_i = sum_c |dO_ic||O_ic|),
    and D uses the forward's bf16 O (at most 2^-9 E_i);
  * dS and P are rounded to bf16 as MFMA operands (2^-9 relative each), and
    every output is rounded to bf16 (2^-9 relative);
  * the products accumulate n terms in fp32 (at most n 2^-24 of the sum of
    |terms|, n = Nk for dQ, the GQA group's rows for dK and dV).
So with U_ij = |dS_ij| (2^-8 + relP_ij) + P_ij (2^-8 E_i + 2 d 2^-24 (A_ij + E_i)):
  |dQ - dQ_ref| <= scale sum_j U_ij |K_j| + 2^-8 |dQ_ref| + Nk 2^-24 scale sum_j |dS_ij||K_j|
  |dK - dK_ref| <= scale sum_i U_ij |Q_i| + 2^-8 |dK_ref| + n 2^-24 scale sum_i |dS_ij||Q_i|
  |dV - dV_ref| <= sum_i P_ij (2^-8 + relP_ij) |dO_i| + 2^-8 |dV_ref| + n 2^-24 sum_i P_ij |dO_i|
elementwise (sums over the GQA group's query heads for dK, dV). Where the
exact gradient vanishes (one visible key: dS = P (dP - D) = 0) the bound
reduces to the fp32 cancellation residue of dP - D. Also: relative
Frobenius error <= 1e-2 where the exact gradient is not zero, and rows with
no visible key get dQ = 0 exactly."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _dev_bf16(seed, t, shape):
    import torch
    bits = synth.draw_bf16(seed, t, shape)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")


def _f64(seed, t, shape):
    return synth.bf16_bits_to_f32(synth.draw_bf16(seed, t, shape)).astype(np.float64)


def _run(w):
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = (_dev_bf16(w.seed, t, s) for t, s in ((0, w.q_shape), (1, w.kv_shape), (2, w.kv_shape)))
    do = _dev_bf16(w.seed, synth.TENSOR_DO, w.q_shape)
    say(f"  launch fa_fwd + fa_bwd {w}")
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def _bounds(w, q, k, v, do):
    """Per-element error bounds for (dQ, dK, dV) and the exact gradients, from
    the oracle's per-head quantities (see the module docstring)."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    u = 2.0 ** -24
    ref = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(k)]
    bnd = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(k)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qh, kh, vh, doh = q[b, h], k[b, g], v[b, g], do[b, h]
            dq, dk, dv, D, P, dP = oracle.attention_backward_head(qh, kh, vh, doh, w.scale, w.causal)
            o = P @ vh
            A = np.abs(doh) @ np.abs(vh).T
            E = (np.abs(doh) * np.abs(o)).sum(axis=1)
            relP = 2.0 ** -16 * w.scale * (np.abs(qh) @ np.abs(kh).T) + 2.0 ** -17
            dS = P * (dP - D[:, None])
            U = np.abs(dS) * (2.0 ** -8 + relP) + P * (2.0 ** -8 * E[:, None] + 2 * d * u * (A + E[:, None]))
            ref[0][b, h] = dq
            ref[1][b, g] += dk
            ref[2][b, g] += dv
            bnd[0][b, h] = (w.scale * (U @ np.abs(kh)) + 2.0 ** -8 * np.abs(dq)
                            + max(Nk, 1) * u * w.scale * (np.abs(dS) @ np.abs(kh)))
            n = max(G * Nq, 1)
            bnd[1][b, g] += w.scale * (U.T @ np.abs(qh)) + n * u * w.scale * (np.abs(dS).T @ np.abs(qh))
            bnd[2][b, g] += (P * (2.0 ** -8 + relP)).T @ np.abs(doh) + n * u * (P.T @ np.abs(doh))
    bnd[1] += 2.0 ** -8 * np.abs(ref[1])
    bnd[2] += 2.0 ** -8 * np.abs(ref[2])
    return ref, bnd


def _check(got, ref, bnd, what):
    for name, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bnd):
        assert not np.isnan(g).any(), f"{what} {name}: NaN"
        if not r.size:
            continue
        err = np.abs(g - r)
        ratio = float(np.max(err / np.maximum(bd, 1e-300)))
        fro = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
        say(f"  {what} {name}: max|d| = {float(err.max()):.3e}, max |d|/bound = {ratio:.3f}, rel-fro {fro:.2e}")
        assert np.all(err <= bd), f"{what} {name}: error above the per-element bound (max ratio {ratio:.3f})"
        if np.linalg.norm(r) > 1e-6 * np.sqrt(r.size):
            assert fro <= 1e-2, f"{what} {name}: relative Frobenius error {fro:.3e}"


CASES = [
    # One key: the exact dQ and dK vanish (dS = dP - D = 0 with P = 1).
    synth.Workload("bwd_one_key_gqa_319_rows", 1, 4, 1, 319, 1, 128, seed=9),
    synth.Workload("bwd_one_key_causal_rows", 2, 2, 2, 40, 1, 64, causal=True, seed=10),
    # Causal with Nq = Nk: row 0 sees exactly one key.
    synth.Workload("bwd_single_visible_key_rows", 1, 2, 1, 70, 70, 128, causal=True, seed=11),
    synth.Workload("bwd_single_head_n256_d64", 1, 1, 1, 256, 256, 64),
    synth.Workload("bwd_single_head_n256_d64_causal", 1, 1, 1, 256, 256, 64, causal=True),
    synth.Workload("bwd_ragged_gqa", 2, 4, 2, 200, 333, 128, seed=1),
    synth.Workload("bwd_ragged_gqa_causal", 2, 4, 2, 200, 333, 128, causal=True, seed=2),
    synth.Workload("bwd_more_queries_than_keys_causal", 1, 3, 1, 300, 70, 128, causal=True, seed=5),
    synth.Workload("bwd_one_query_one_key", 1, 1, 1, 1, 1, 128),
    synth.Workload("bwd_keys_below_one_block", 1, 2, 2, 150, 17, 128, seed=4),
    synth.Workload("bwd_gqa_8to1_d64_causal", 1, 8, 1, 130, 190, 64, causal=True, seed=6),
    # Tails one row / one key past a block edge (the second wave of a pair
    # then holds a single valid row or key), and a causal diagonal offset.
    synth.Workload("bwd_gqa_4to1_d128_tail_129", 1, 8, 2, 129, 129, 128, seed=7),
    synth.Workload("bwd_gqa_4to1_d128_causal_65x257", 2, 8, 2, 65, 257, 128, causal=True, seed=8),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_bwd_full_oracle(w):
    say(f"case bwd full {w.name}")
    got = _run(w)
    q, k, v = synth.inputs_f64(w)
    do = _f64(w.seed, synth.TENSOR_DO, w.q_shape)
    ref, bnd = _bounds(w, q, k, v, do)
    _check(got, ref, bnd, w.name)
    if w.causal and w.Nq > w.Nk:
        assert np.all(got[0][:, :, : w.Nq - w.Nk] == 0.0), "rows without keys must get dQ = 0"


def _random_shapes(n=24, seed=2026):
    """Seeded mixed shapes: batch 1-2, 1-3 KV heads, GQA 1/2/4, 1..399 rows and
    keys, d 64 or 128, with and without causal."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append(synth.Workload(f"bwd_random_{i}", int(rng.integers(1, 3)), hq, hkv, int(rng.integers(1, 400)),
                                  int(rng.integers(1, 400)), d, causal=bool(rng.integers(0, 2)), seed=200 + i))
    return out


@pytest.mark.parametrize("w", _random_shapes(), ids=lambda w: w.name)
def test_bwd_random_shapes(w):
    say(f"case bwd random {w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} {w.Nq}x{w.Nk} d{w.d} causal={w.causal}")
    got = _run(w)
    q, k, v = synth.inputs_f64(w)
    do = _f64(w.seed, synth.TENSOR_DO, w.q_shape)
    ref, bnd = _bounds(w, q, k, v, do)
    _check(got, ref, bnd, w.name)


@pytest.mark.parametrize("name", ["batched", "batched_causal", "pages_shape"])
def test_bwd_full_size_heads(name):
    """Full-size launches: the batched shape (B4 H16 2048^2 d128), with and
    without causal, and the pages' shape (B1 H8 4096 x 8192, the benchmark's
    backward); the oracle computes two whole heads (MHA: heads are
    independent)."""
    if name == "pages_shape":
        w = synth.WORKLOADS["pages_shape_h8_q4096_kv8192"]
    else:
        w = synth.Workload("bwd_batched_b4h16_n2048", 4, 16, 16, 2048, 2048, 128, causal=name.endswith("causal"))
    causal = w.causal
    say(f"case bwd full-size {w.name} causal={causal}")
    got = _run(w)
    for (b, h) in ((0, 0), (w.B - 1, w.Hq - 1)):
        q, k, v = synth.inputs_f64(w, q_heads=[(b, h)], kv_heads=[(b, h)])
        do = synth.bf16_bits_to_f32(synth.draw_bf16(w.seed, synth.TENSOR_DO, w.q_shape, heads=[(b, h)]))
        do = do.astype(np.float64)
        wh = synth.Workload(w.name, 1, 1, 1, w.Nq, w.Nk, w.d, causal=causal, seed=w.seed)
        ref, bnd = _bounds(wh, q[:, None], k[:, None], v[:, None], do[:, None])
        _check([g[b:b + 1, h:h + 1] for g in got], ref, bnd, f"{w.name} head ({b},{h})")


def test_bwd_degenerate_sizes():
    """Nq = 0: no query, so dK = dV = 0; Nk = 0: no key, so dQ = 0 (the
    forward gives O = 0 and LSE = -inf)."""
    import torch
    import exact_io_aware_17_amd as fa
    for (nq, nk) in ((0, 70), (50, 0)):
        w = synth.Workload(f"bwd_degenerate_{nq}_{nk}", 1, 2, 1, nq, nk, 128, causal=True)
        say(f"case bwd degenerate Nq={nq} Nk={nk}")
        q, k, v = (_dev_bf16(w.seed, t, s) for t, s in ((0, w.q_shape), (1, w.kv_shape), (2, w.kv_shape)))
        do = _dev_bf16(w.seed, synth.TENSOR_DO, w.q_shape)
        o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True, scale=w.scale)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert t.numel() == 0 or float(t.float().abs().max()) == 0.0


def test_bwd_deterministic():
    """Every gradient element is written once by one lane (no atomics), so two
    calls on the same inputs agree bit for bit."""
    import torch
    import exact_io_aware_17_amd as fa
    w = synth.Workload("bwd_determinism", 2, 4, 2, 300, 517, 128, causal=True)
    say("case bwd determinism")
    q, k, v = (_dev_bf16(w.seed, t, s) for t, s in ((0, w.q_shape), (1, w.kv_shape), (2, w.kv_shape)))
    do = _dev_bf16(w.seed, synth.TENSOR_DO, w.q_shape)
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    first = fa.backward(q, k, v, o, lse, do, causal=True, scale=w.scale)
    second = fa.backward(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
