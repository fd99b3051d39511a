"""Race check of the LDS tile pipelines: the library built with FA_LDS_POISON,
in which every tile copy first fills the LDS bytes it will write with NaN
(all-ones: NaN in bf16, fp32 and E4M3). A read that runs ahead of a copy's
wait and barrier, or lags behind the next copy into its slot, then reads NaN,
which propagates into O; parity against the oracle on ragged, causal, GQA,
head size 64/128/192/256, every layout of the d = 64/128 kernel, fp8 and
full-size launches shows that no read does."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, device_inputs, errors, oracle_full, oracle_sample, sample_rows, say
import test_parity_fp8_gpu as fp8_tests
from test_parity_gpu import ROW_GROUPS

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module")
def fa_poison():
    import exact_io_aware_17_amd as fa
    from exact_io_aware_17_amd.build import POISON_LIB_PATH
    saved = (fa.LIB_PATH, fa._lib)
    fa.LIB_PATH, fa._lib = POISON_LIB_PATH, None
    fa.lib()
    yield fa
    fa.LIB_PATH, fa._lib = saved


def _run(fa, w):
    import torch
    q, k, v = device_inputs(w)
    say(f"  poison build: fa_fwd {w}")
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    synth.Workload("poison_ragged_gqa", 2, 4, 2, 200, 333, 128),
    synth.Workload("poison_ragged_gqa_causal", 2, 4, 2, 200, 333, 128, causal=True),
    synth.Workload("poison_causal_d64", 2, 2, 1, 257, 257, 64, causal=True, seed=3),
    synth.Workload("poison_queries_over_keys_causal", 1, 3, 1, 300, 70, 128, causal=True, seed=5),
    synth.Workload("poison_keys_below_one_tile", 1, 2, 2, 300, 17, 128),
    synth.Workload("poison_long_keys", 1, 2, 1, 130, 1500, 128, seed=9),
    synth.Workload("poison_d256_causal", 1, 2, 2, 384, 384, 256, causal=True),
    synth.Workload("poison_d256_ragged_gqa", 2, 4, 2, 200, 333, 256, seed=1),
    synth.Workload("poison_d192_ragged_gqa_causal", 2, 4, 2, 200, 333, 192, causal=True, seed=12),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_poison_bf16_full_oracle(fa_poison, w):
    o, lse = _run(fa_poison, w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name + " (poison build)")


@pytest.mark.parametrize("w", ROW_GROUPS, ids=lambda w: w.name)
def test_poison_bf16_row_groups(fa_poison, w):
    """The row-group layouts (both wave groups on their own rows, single
    blocks and causal pairs) at sizes the oracle covers whole."""
    assert fa_poison.fa_fwd_layout(w.B, w.Hq, w.Nq, w.d, w.causal).startswith("rows")
    o, lse = _run(fa_poison, w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name + " (poison build)")


@pytest.mark.parametrize("w", fp8_tests.SMALL, ids=lambda w: w.name)
def test_poison_fp8_cases(fa_poison, w):
    """The fp8 parity cases (ragged, causal, GQA, one key, one query) with
    their per-element E4M3 bound, on the poison build."""
    fp8_tests.test_fp8_full_oracle(w)


@pytest.mark.parametrize("name", ["pages_shape_h8_q4096_kv8192", "batched_prefill_b4h16_n2048_causal"])
def test_poison_full_size(fa_poison, name):
    w = W[name]
    o, lse = _run(fa_poison, w)
    assert np.isfinite(o).all() and not np.isnan(lse).any(), "NaN in a full-size launch of the poison build"
    heads = [(0, 0), (w.B - 1, w.Hq - 1)]
    rows = sample_rows(w.Nq)
    o_ref, lse_ref = oracle_sample(w, heads, rows)
    for n, (b, h) in enumerate(heads):
        assert_close(errors(o[b, h, rows], o_ref[n], lse[b, h, rows], lse_ref[n]), what=f"{name} head {h} (poison)")


def test_poison_fp8(fa_poison):
    import torch
    w = synth.Workload("poison_fp8_causal", 1, 4, 2, 300, 517, 128, causal=True, seed=4)
    q8, k8, v8 = (torch.from_numpy(synth.draw_e4m3(w.seed, t, s)).to("cuda")
                  for t, s in ((0, w.q_shape), (1, w.kv_shape), (2, w.kv_shape)))
    say("  poison build: fa_fwd_fp8 causal 300x517 GQA")
    o, lse = fa_poison.forward_fp8(q8, k8, v8, synth.FP8_DESCALE, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fp8(q8.cpu().numpy(), k8.cpu().numpy(), v8.cpu().numpy(), synth.FP8_DESCALE,
                                        w.scale, True)
    o = o.float().cpu().numpy()
    assert np.isfinite(o).all()
    fin = np.isfinite(l_ref)
    assert float(np.max(np.abs(lse.cpu().numpy()[fin] - l_ref[fin]))) <= 1e-3
    # E4M3 probabilities: each O element within 2^-4 of sum_j P_ij |V_j| (bounded by 2^-4 max|V| here).
    assert float(np.max(np.abs(o - o_ref))) <= 2.0 ** -4 * 6.25 + 1e-3
