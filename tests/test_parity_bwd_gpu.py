"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 oracle (oracle.attention_backward) on the same seeded bf16 inputs.

Tolerance, derived from the arithmetic (the task fixes none for gradients):
every product runs on bf16 operands with fp32 accumulation; P and dS are
rounded to bf16 (2^-9 relative per term) before dV = P^T dO, dK = dS^T Q and
dQ = dS K; the outputs are rounded to bf16 (2^-9 relative); D = rowsum(dO O)
uses the forward's bf16 O, which moves dS by about 2^-9 |dO||O|, small
against |dP - D|. Sums of such terms keep the relative error near 2^-9 of
sum |terms|, so per tensor: max |G - G_ref| <= 2e-2 max |G_ref| + 1e-6 and
||G - G_ref||_F <= 1e-2 ||G_ref||_F (1e-6 per element where G_ref is zero,
e.g. dQ and dK with a single key, where dS = dP - D vanishes exactly and the
GPU keeps only fp32 summation-order residue). Rows with no visible key must
get dQ = 0 exactly."""
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


def _check(got, ref, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert not np.isnan(g).any(), f"{what} {name}: NaN"
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        e_max = float(np.max(np.abs(g - r))) if r.size else 0.0
        fro = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)) if r.size else 0.0
        say(f"  {what} {name}: max|d| = {e_max:.3e} ({e_max / max(scale, 1e-30):.2e} of max|ref|), rel-fro {fro:.2e}")
        assert e_max <= 2e-2 * scale + 1e-6, f"{what} {name}: max error {e_max:.3e} > 2e-2 * {scale:.3e} + 1e-6"
        if np.linalg.norm(r) > 0:
            assert fro <= 1e-2, f"{what} {name}: relative Frobenius error {fro:.3e}"
        else:
            assert float(np.linalg.norm(g)) <= 1e-6 * np.sqrt(g.size), f"{what} {name}: nonzero gradient"


CASES = [
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
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, w.scale, w.causal)
    _check(got, (dq, dk, dv), w.name)
    if w.causal and w.Nq > w.Nk:
        assert np.all(got[0][:, :, : w.Nq - w.Nk] == 0.0), "rows without keys must get dQ = 0"


def _random_shapes(n=24, seed=2026):
    """Seeded mixed shapes: batch 1-2, 1-3 KV heads, GQA 1/2/4, 2..399 rows and
    keys (at least two keys, so that no gradient is exactly zero), d 64 or
    128, with and without causal."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append(synth.Workload(f"bwd_random_{i}", int(rng.integers(1, 3)), hq, hkv, int(rng.integers(2, 400)),
                                  int(rng.integers(2, 400)), d, causal=bool(rng.integers(0, 2)), seed=200 + i))
    return out


@pytest.mark.parametrize("w", _random_shapes(), ids=lambda w: w.name)
def test_bwd_random_shapes(w):
    say(f"case bwd random {w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} {w.Nq}x{w.Nk} d{w.d} causal={w.causal}")
    got = _run(w)
    q, k, v = synth.inputs_f64(w)
    do = _f64(w.seed, synth.TENSOR_DO, w.q_shape)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, w.scale, w.causal)
    _check(got, (dq, dk, dv), w.name)


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
        dq, dk, dv, _ = oracle.attention_backward(q[:, None], k[:, None], v[:, None], do[:, None], w.scale, causal)
        _check([g[b:b + 1, h:h + 1] for g in got], (dq, dk, dv), f"{w.name} head ({b},{h})")


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
