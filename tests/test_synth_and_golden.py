"""Seeded input generator and the pages' benchmark-table fixture (CPU only)."""
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_benchmark_5090.txt")


def test_bf16_rounding_matches_torch():
    """The bit formula is round-to-nearest-even: compare with torch's fp32->bf16
    conversion on random values and on exact ties."""
    r = np.random.default_rng(0)
    x = r.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** r.integers(-5, 5, 100000)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x.astype(np.float32), ties, -ties, np.float32([0.0, -0.0, 1.0, 3.0e38])])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_deterministic_and_slab_local():
    shape = (2, 3, 17, 8)
    a = synth.draw(0, synth.TENSOR_K, shape)
    b = synth.draw(0, synth.TENSOR_K, shape)
    np.testing.assert_array_equal(a, b)
    assert a.shape == shape and a.dtype == np.float32
    one = synth.draw(0, synth.TENSOR_K, shape, heads=[(1, 2)], rows=np.array([3, 16]))
    np.testing.assert_array_equal(one[0], a[1, 2, [3, 16]])
    c = synth.draw(0, synth.TENSOR_V, shape)
    assert not np.array_equal(a, c)
    bits = synth.draw_bf16(0, synth.TENSOR_K, shape)
    np.testing.assert_array_equal(bits, synth.bf16_bits(a))


def test_inputs_f64_exact_widening():
    w = synth.WORKLOADS["single_head_n256_d64"]
    q, k, v = synth.inputs_f64(w)
    assert q.shape == (1, 1, 256, 64) and k.shape == (1, 1, 256, 64)
    assert np.array_equal(q.astype(np.float32).astype(np.float64), q)
    # bf16 values carry at most 8 significant bits.
    m, _ = np.frexp(q)
    assert np.all((m * 256) == np.round(m * 256))
    qf, _, _ = synth.inputs_f64(w, bf16=False)
    assert np.max(np.abs(qf - q)) <= np.max(np.abs(qf)) * 2.0 ** -8


def _golden():
    rows = {}
    sol = None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("sol_tflops"):
            sol = float(line.split()[1])
        elif line.startswith("shape"):
            shape = dict(kv.split("=") for kv in line.split()[1:])
        else:
            name, tf, pct = line.split("|")
            rows[name] = (float(tf), float(pct))
    return sol, shape, rows


def test_pages_table_sol_convention():
    """%SOL on the page is TFLOPS / 209.5 for every row, to the printed 2 decimals."""
    sol, _, rows = _golden()
    assert sol == 209.5 and len(rows) == 8
    for name, (tf, pct) in rows.items():
        assert abs(100.0 * tf / sol - pct) <= 0.006, name


def test_pages_shape_is_the_benchmark_workload():
    _, shape, _ = _golden()
    w = synth.WORKLOADS["pages_shape_h8_q4096_kv8192"]
    assert (w.B, w.Hq, w.Nq, w.Nk, w.d) == (int(shape["bs"]), int(shape["heads"]), int(shape["q"]),
                                             int(shape["kv"]), int(shape["head_dim"]))
    assert not w.causal
    assert w.flops() == pytest.approx(137.438953472e9)
    # The page's best hand kernel (v5) would take about 0.695 ms at this count.
    assert w.flops() / 197.74e12 == pytest.approx(0.000695, rel=1e-3)


def test_workload_byte_and_flop_formulas():
    w = synth.WORKLOADS["gqa_decode_b64_hq32_hkv8_kv8192"]
    assert w.algorithmic_bytes() == 2 * 2**30 + 2 * 2**19 + 8192
    c = synth.WORKLOADS["long_causal_h32_n16384"]
    assert c.flops() == 4.0 * 32 * 16384 * 16384 * 128 / 2
