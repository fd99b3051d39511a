"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Tolerances: max|O - O_ref| <= 2e-2 and max|LSE - LSE_ref|
<= 1e-3 for bf16 inputs with fp32 accumulation; 1e-5 for the fp32 path."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (F32_TOL, assert_close, device_inputs, errors, oracle_full, oracle_sample,
                         paged_device, paged_numpy, sample_rows, say)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _fa():
    import exact_io_aware_17_amd as fa
    fa.lib()
    return fa


def _run_fwd(w, fp32=False):
    import torch
    fa = _fa()
    q, k, v = device_inputs(w, bf16=not fp32)
    say(f"  launch {'fa_fwd_fp32' if fp32 else 'fa_fwd'} {w}")
    if fp32:
        o, lse = fa.forward_fp32(q, k, v, causal=w.causal, scale=w.scale)
    else:
        o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


SMALL = [
    W["single_head_n256_d64"],
    synth.Workload("ragged_gqa", 2, 4, 2, 200, 333, 128),
    synth.Workload("ragged_gqa_causal", 2, 4, 2, 200, 333, 128, causal=True),
    synth.Workload("more_queries_than_keys_causal_d64", 1, 3, 1, 130, 70, 64, causal=True),
    # Head dim 128, causal, Nq > Nk: the first workgroups see no key at all.
    synth.Workload("more_queries_than_keys_causal_d128", 1, 3, 1, 300, 70, 128, causal=True, seed=5),
    synth.Workload("whole_tiles_queries_over_keys_causal", 1, 2, 1, 200, 64, 128, causal=True, seed=6),
    # Exactly one 32-key tile: the second key group has no tile.
    synth.Workload("exactly_one_small_tile", 1, 2, 2, 64, 32, 128, seed=7),
    synth.Workload("one_query_one_key", 1, 1, 1, 1, 1, 128),
    synth.Workload("keys_below_one_tile", 1, 2, 2, 300, 17, 128),
    synth.Workload("square_causal_3_tiles", 1, 2, 2, 384, 384, 128, causal=True),
    synth.Workload("causal_d64_ragged", 2, 2, 1, 257, 257, 64, causal=True, seed=3),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_bf16_full_oracle(w):
    say(f"case bf16 full {w.name}")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name)


# Grids of at least 256 blocks of 256 query rows (pairs of blocks under the
# causal mask) take the row-group layout of the d = 64/128 kernel (both wave
# groups on their own rows, every KV tile): many small heads keep the oracle
# cheap while the launch uses that layout.
ROW_GROUPS = [
    synth.Workload("rows_ragged_gqa", 2, 128, 32, 200, 333, 128, seed=21),
    # 3 blocks per head: pairs (2, 0) and the middle block 1 alone.
    synth.Workload("rows_ragged_gqa_causal_odd_blocks", 2, 128, 32, 600, 650, 128, causal=True, seed=22),
    # Nq > Nk under the mask: the first rows see no key.
    synth.Workload("rows_more_queries_than_keys_causal", 1, 256, 64, 300, 70, 128, causal=True, seed=23),
    synth.Workload("rows_causal_d64", 1, 256, 64, 257, 257, 64, causal=True, seed=24),
    synth.Workload("rows_d64_long_keys", 1, 256, 256, 100, 1000, 64, seed=25),
    synth.Workload("rows_keys_below_one_tile", 1, 256, 128, 256, 17, 128, seed=26),
    # One query per head: seven of the eight waves hold no row.
    synth.Workload("rows_one_query", 4, 64, 16, 1, 1000, 128, seed=27),
]


@pytest.mark.parametrize("w", ROW_GROUPS, ids=lambda w: w.name)
def test_bf16_row_groups_full_oracle(w):
    say(f"case bf16 row groups {w.name}")
    assert _fa().fa_fwd_layout(w.B, w.Hq, w.Nq, w.d, w.causal).startswith("rows")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name)


def _random_row_group_shapes(n=12, seed=2031):
    """Seeded shapes whose grids take the row-group layouts: batch 1-2, 16,
    32 or 64 KV heads with GQA 1/2/4, 1..519 rows and keys, d 64 or 128,
    causal or not, kept only if there are at least 256 blocks of 256 rows
    (or causal pairs of them)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([16, 32, 64]))
        hq = hkv * int(rng.choice([1, 2, 4]))
        b, nq, nk, causal = int(rng.integers(1, 3)), int(rng.integers(1, 520)), int(rng.integers(1, 520)), bool(rng.integers(0, 2))
        blocks = -(-nq // 256)
        units = (blocks + 1) // 2 if causal and blocks >= 2 else blocks
        if b * hq * units < 256:
            continue
        out.append(synth.Workload(f"rows_random_{len(out)}", b, hq, hkv, nq, nk, d, causal=causal, seed=400 + len(out)))
    return out


@pytest.mark.parametrize("w", _random_row_group_shapes(), ids=lambda w: w.name)
def test_bf16_row_groups_random_shapes(w):
    say(f"case bf16 row groups random {w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} {w.Nq}x{w.Nk} d{w.d} causal={w.causal}")
    assert _fa().fa_fwd_layout(w.B, w.Hq, w.Nq, w.d, w.causal).startswith("rows")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name)


def _random_shapes(n=24, seed=2027):
    """Seeded mixed shapes: batch 1-2, 1-3 KV heads, GQA 1/2/4, 1..399 rows and
    keys, d 64, 128 or 256, with and without causal."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.integers(1, 4))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append(synth.Workload(f"fwd_random_{i}", int(rng.integers(1, 3)), hq, hkv, int(rng.integers(1, 400)),
                                  int(rng.integers(1, 400)), d, causal=bool(rng.integers(0, 2)), seed=300 + i))
    return out


@pytest.mark.parametrize("w", _random_shapes(), ids=lambda w: w.name)
def test_bf16_random_shapes(w):
    say(f"case bf16 random {w.name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} {w.Nq}x{w.Nk} d{w.d} causal={w.causal}")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fp32_full_oracle(w):
    say(f"case fp32 full {w.name}")
    o, lse = _run_fwd(w, fp32=True)
    o_ref, lse_ref = oracle_full(w, bf16=False)
    assert_close(errors(o, o_ref, lse, lse_ref), F32_TOL, F32_TOL, what=w.name + " fp32", o_fro_tol=F32_TOL)


D256 = [
    synth.Workload("d256_single_head_n256", 1, 1, 1, 256, 256, 256),
    synth.Workload("d256_ragged_gqa", 2, 4, 2, 200, 333, 256, seed=1),
    synth.Workload("d256_ragged_gqa_causal", 2, 4, 2, 200, 333, 256, causal=True, seed=2),
    synth.Workload("d256_more_queries_than_keys_causal", 1, 3, 1, 300, 70, 256, causal=True, seed=5),
    synth.Workload("d256_one_query_one_key", 1, 1, 1, 1, 1, 256),
    synth.Workload("d256_keys_below_one_tile", 1, 2, 2, 300, 17, 256, seed=4),
    synth.Workload("d256_square_causal", 1, 2, 2, 384, 384, 256, causal=True),
    synth.Workload("d256_odd_tiles_causal", 1, 2, 1, 161, 161, 256, causal=True, seed=6),
    # 8 x 64 heads x 2 query blocks = 1024 workgroups: the one-group layout.
    synth.Workload("d256_many_blocks_gqa_causal_ragged", 8, 64, 8, 130, 77, 256, causal=True, seed=7),
    synth.Workload("d256_many_blocks_ragged", 4, 64, 16, 200, 90, 256, seed=8),
    # Head size 192 (384-byte rows, 24 chunks: a copy instruction covers 2 2/3
    # rows, and the swizzle works within groups of 8 chunks).
    synth.Workload("d192_single_head_n256", 1, 1, 1, 256, 256, 192),
    synth.Workload("d192_ragged_gqa", 2, 4, 2, 200, 333, 192, seed=11),
    synth.Workload("d192_ragged_gqa_causal", 2, 4, 2, 200, 333, 192, causal=True, seed=12),
    synth.Workload("d192_more_queries_than_keys_causal", 1, 3, 1, 300, 70, 192, causal=True, seed=13),
    synth.Workload("d192_one_query_one_key", 1, 1, 1, 1, 1, 192),
    synth.Workload("d192_keys_below_one_tile", 1, 2, 2, 300, 17, 192, seed=14),
    synth.Workload("d192_odd_tiles_causal", 1, 2, 1, 161, 161, 192, causal=True, seed=15),
    synth.Workload("d192_many_blocks_gqa_causal_ragged", 8, 64, 8, 130, 77, 192, causal=True, seed=16),
]


@pytest.mark.parametrize("w", D256, ids=lambda w: w.name)
def test_bf16_d256_full_oracle(w):
    """Head size 256 (fa_fwd's d = 256 kernel) against the oracle."""
    say(f"case bf16 d256 full {w.name}")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    assert_close(errors(o, o_ref, lse, lse_ref), what=w.name)


@pytest.mark.parametrize("name", ["pages_shape_d256_h8_q4096_kv8192", "batched_d256_b4h16_n2048",
                                  "batched_d256_b4h16_n2048_causal", "pages_shape_d192_h8_q4096_kv8192",
                                  "batched_d192_b4h16_n2048_causal"])
def test_bf16_d256_full_size_sampled(name):
    """Full-size d = 256 and d = 192 launches: the pages' shape (256
    workgroups, the two-group layout) and the batched shape (1024, the
    one-group layout)."""
    d = 192 if "d192" in name else 256
    w = W.get(name) or synth.Workload(name, 4, 16, 16, 2048, 2048, d, causal=name.endswith("causal"))
    say(f"case bf16 d256 full-size {w.name}")
    o, lse = _run_fwd(w)
    rows = sample_rows(w.Nq)
    heads = [(0, 0), (w.B - 1, w.Hq - 3)]
    o_ref, lse_ref = oracle_sample(w, heads, rows)
    for n, (b, h) in enumerate(heads):
        assert_close(errors(o[b, h, rows], o_ref[n], lse[b, h, rows], lse_ref[n]), what=f"{w.name} head {h}")


@pytest.mark.parametrize("name", ["batched_prefill_b4h16_n2048", "batched_prefill_b4h16_n2048_causal",
                                  "pages_shape_h8_q4096_kv8192"])
def test_bf16_full_size_every_element(name):
    """Full-size launch (the configuration the benchmark times: the pages'
    shape in KV-parity blocks, the batched shapes in row groups), every
    element of every head against the oracle."""
    w = W[name]
    layout = _fa().fa_fwd_layout(w.B, w.Hq, w.Nq, w.d, w.causal)
    assert layout == {"pages_shape_h8_q4096_kv8192": "kv_parity", "batched_prefill_b4h16_n2048": "rows",
                      "batched_prefill_b4h16_n2048_causal": "rows_paired"}[name]
    say(f"case bf16 full-size {name} ({layout}), every head")
    o, lse = _run_fwd(w)
    o_ref, lse_ref = oracle_full(w)
    for b in range(w.B):
        for h in range(w.Hq):
            assert_close(errors(o[b, h], o_ref[b, h], lse[b, h], lse_ref[b, h]), what=f"{name} ({b},{h})")
    assert_close(errors(o, o_ref, lse, lse_ref), what=f"{name} all heads")


def test_bf16_long_causal_whole_heads():
    """The long causal workload (B1 H32 16384^2) at full size: four whole heads
    (first, last and two between) against the oracle, every row."""
    w = W["long_causal_h32_n16384"]
    say("case bf16 full-size long causal, 4 whole heads")
    o, lse = _run_fwd(w)
    heads = [(0, 0), (0, 9), (0, 22), (0, 31)]
    rows = np.arange(w.Nq)
    o_ref, lse_ref = oracle_sample(w, heads, rows)
    for n, (b, h) in enumerate(heads):
        assert_close(errors(o[b, h], o_ref[n], lse[b, h], lse_ref[n]), what=f"long causal head {h}")
    assert np.isfinite(lse).all() and np.isfinite(o).all()


def test_fp32_batched_sampled():
    w = W["batched_prefill_b4h16_n2048_causal"]
    say("case fp32 full-size batched causal")
    o, lse = _run_fwd(w, fp32=True)
    heads = [(0, 0), (3, 15)]
    rows = sample_rows(w.Nq, n_random=8)
    o_ref, lse_ref = oracle_sample(w, heads, rows, bf16=False)
    got_o = np.stack([o[b, h][rows] for (b, h) in heads])
    got_l = np.stack([lse[b, h][rows] for (b, h) in heads])
    assert_close(errors(got_o, o_ref, got_l, lse_ref), F32_TOL, F32_TOL, what="fp32 batched causal",
                 o_fro_tol=F32_TOL)


def _run_decode(w, fetch_partials=False):
    import torch
    fa = _fa()
    q, k, v = device_inputs(w)
    ws = fa.workspace_for(q, w.num_splits)
    say(f"  launch fa_fwd_splitkv {w}")
    o, lse = fa.decode(q, k, v, w.num_splits, causal=w.causal, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    out = (o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    if fetch_partials:
        op, lp = fa.split_views(ws, w.B, w.Hq, w.Nq, w.d, w.num_splits)
        out = out + (op.cpu().numpy().astype(np.float64), lp.cpu().numpy().astype(np.float64))
    return out


def test_decode_full_size():
    """GQA split-KV decode at full size; oracle on every row of three batches,
    for both the merged result and the per-chunk partials."""
    w = W["gqa_decode_b64_hq32_hkv8_kv8192"]
    say("case decode full-size")
    o, lse, op, lp = _run_decode(w, fetch_partials=True)
    group = w.Hq // w.Hkv
    for b in (0, 37, 63):
        q, k, v = synth.inputs_f64(w, q_heads=[(b, h) for h in range(w.Hq)],
                                   kv_heads=[(b, g) for g in range(w.Hkv)])
        q4 = q[None]
        k4 = k[None]
        v4 = v[None]
        o_ref, l_ref = oracle.attention(q4, k4, v4, w.scale, False)
        assert_close(errors(o[b], o_ref[0], lse[b], l_ref[0]), what=f"decode b={b}")
        op_ref, lp_ref = oracle.splitkv_partials(q4, k4, v4, w.scale, w.num_splits)
        e = errors(op[b], op_ref[0], lp[b], lp_ref[0])
        assert_close(e, what=f"decode partials b={b}")
        assert group == 4


DECODE_EDGE = [
    synth.Workload("nondividing_splits", 2, 8, 2, 1, 1000, 128, num_splits=7),
    synth.Workload("one_split", 1, 4, 4, 1, 777, 128, num_splits=1),
    synth.Workload("more_splits_than_keys", 1, 4, 1, 1, 5, 128, num_splits=9),
    synth.Workload("multi_query_causal", 2, 6, 2, 3, 300, 128, causal=True, num_splits=4),
    synth.Workload("decode_d64_gqa8", 3, 16, 2, 1, 2048, 64, num_splits=16),
    synth.Workload("rows_over_32", 1, 40, 1, 2, 513, 128, num_splits=3),
]


@pytest.mark.parametrize("w", DECODE_EDGE, ids=lambda w: w.name)
def test_decode_edge_cases(w):
    say(f"case decode {w.name}")
    o, lse, op, lp = _run_decode(w, fetch_partials=True)
    q, k, v = synth.inputs_f64(w)
    o_ref, l_ref = oracle.attention(q, k, v, w.scale, w.causal)
    assert_close(errors(o, o_ref, lse, l_ref), what=w.name)
    op_ref, lp_ref = oracle.splitkv_partials(q, k, v, w.scale, w.num_splits, w.causal)
    assert_close(errors(op, op_ref, lp, lp_ref), what=w.name + " partials")


# Paged K/V: (workload for the shapes, per-sequence key counts, page size).
PAGED = [
    (synth.Workload("paged16_gqa", 3, 8, 2, 1, 1000, 128, num_splits=4), [1000, 1, 517], 16),
    (synth.Workload("paged64_multiquery_causal", 3, 6, 2, 3, 300, 128, causal=True, num_splits=3, seed=8),
     [300, 64, 129], 64),
    (synth.Workload("paged32_d64_empty_sequence", 3, 4, 4, 1, 200, 64, num_splits=7, seed=9), [200, 0, 33], 32),
    (synth.Workload("paged256_causal_two_chunks", 2, 4, 1, 2, 700, 128, causal=True, num_splits=2, seed=10),
     [700, 256], 256),
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: c[0].name)
def test_paged_decode(case):
    """fa_fwd_splitkv_paged on a randomly permuted page cache against the
    paged oracle (each sequence its own key count)."""
    import torch
    fa = _fa()
    w, lens, page = case
    q, k, v = device_inputs(w)
    kc, vc, table = paged_device(k, v, page, seed=w.seed + page)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    say(f"case paged decode {w.name} page={page} lens={lens}")
    o, lse = fa.decode_paged(q, kc, vc, table, sl, w.num_splits, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    q64, k64, v64 = synth.inputs_f64(w)
    kc64, vc64, table64 = paged_numpy(k64, v64, page, seed=w.seed + page)
    assert np.array_equal(table64, table.cpu().numpy())
    o_ref, l_ref = oracle.paged_attention(q64, kc64, vc64, table64, lens, w.scale, w.causal)
    o_got = o.float().cpu().numpy().astype(np.float64)
    l_got = lse.cpu().numpy().astype(np.float64)
    assert_close(errors(o_got, o_ref, l_got, l_ref), what=w.name)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o_got[b] == 0) and np.all(np.isneginf(l_got[b]))


def test_paged_identity_layout_matches_contiguous():
    """Pages laid out in order (page j of sequence b at b * pages + j) give
    bit-identical results to the contiguous split-KV path."""
    import torch
    fa = _fa()
    w = synth.Workload("paged_identity", 2, 8, 2, 1, 1024, 128, num_splits=5, seed=12)
    q, k, v = device_inputs(w)
    page, mp = 16, 1024 // 16
    kc = k.reshape(2, 2, mp, page, 128).permute(0, 2, 1, 3, 4).reshape(2 * mp, 2, page, 128).contiguous()
    vc = v.reshape(2, 2, mp, page, 128).permute(0, 2, 1, 3, 4).reshape(2 * mp, 2, page, 128).contiguous()
    table = torch.arange(2 * mp, dtype=torch.int32, device="cuda").reshape(2, mp)
    sl = torch.full((2,), 1024, dtype=torch.int32, device="cuda")
    say("case paged identity layout")
    o1, l1 = fa.decode_paged(q, kc, vc, table, sl, w.num_splits, scale=w.scale)
    o2, l2 = fa.decode(q, k, v, w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_decode_full_size():
    """The benchmark's paged decode (GQA decode workload, 16-key pages in a
    random order); oracle on every row of three batches."""
    import torch
    fa = _fa()
    w = W["gqa_decode_b64_hq32_hkv8_kv8192"]
    q, k, v = device_inputs(w)
    kc, vc, table = paged_device(k, v, 16, seed=w.seed + 16)
    del k, v
    sl = torch.full((w.B,), w.Nk, dtype=torch.int32, device="cuda")
    say("case paged decode full-size")
    o, lse = fa.decode_paged(q, kc, vc, table, sl, w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    for b in (0, 31, 63):
        q64, k64, v64 = synth.inputs_f64(w, q_heads=[(b, h) for h in range(w.Hq)],
                                         kv_heads=[(b, g) for g in range(w.Hkv)])
        o_ref, l_ref = oracle.attention(q64[None], k64[None], v64[None], w.scale, False)
        assert_close(errors(o[b], o_ref[0], lse[b], l_ref[0]), what=f"paged decode b={b}")


@pytest.mark.parametrize("S,d", [(5, 128), (64, 128), (100, 128), (7, 64), (70, 64)])
def test_combine_entry_point(S, d):
    """fa_combine alone, on seeded random partials (some chunks empty); up to
    64 chunks take the lane-parallel path, more the plain loop."""
    import torch
    fa = _fa()
    r = np.random.default_rng(5 + S)
    B, Hq, Nq = 2, 3, 4
    op = r.standard_normal((B, Hq, S, Nq, d)).astype(np.float32)
    lp = (r.standard_normal((B, Hq, S, Nq)) * 3).astype(np.float32)
    lp[0, 0, 1] = -np.inf
    lp[1, 2, :, 0] = -np.inf   # a row whose chunks are all empty
    op[1, 2, :, 0] = 0.0
    o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    say("case fa_combine")
    fa.fa_combine(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda(), o, lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.combine(op.astype(np.float64), lp.astype(np.float64))
    assert_close(errors(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), l_ref), what="combine")
    assert np.all(o[1, 2, 0].float().cpu().numpy() == 0)


def _bf16_dev(x):
    import torch
    return torch.from_numpy(synth.bf16_bits(x.astype(np.float32)).view(np.int16)).view(torch.bfloat16).cuda()


def test_structured_inputs():
    """Closed forms on the GPU: identical keys give the column mean of V, a
    one-hot query with a large logit selects one V row, V = 1 gives O = 1."""
    import torch
    fa = _fa()
    r = np.random.default_rng(9)
    Nq, Nk, d = 130, 300, 128
    q = r.standard_normal((1, 2, Nq, d))
    krow = r.standard_normal(d)
    k = np.broadcast_to(krow, (1, 2, Nk, d)).copy()
    v = r.standard_normal((1, 2, Nk, d))
    qb, kb, vb = (_bf16_dev(x) for x in (q, k, v))
    say("case structured identical keys")
    o, lse = fa.forward(qb, kb, vb, scale=0.088388346)
    torch.cuda.synchronize()
    vv = vb.float().cpu().numpy().astype(np.float64)
    o_exp = np.broadcast_to(vv.mean(axis=2, keepdims=True), o.shape)
    assert np.max(np.abs(o.float().cpu().numpy() - o_exp)) <= 1e-2
    qq = qb.float().cpu().numpy().astype(np.float64)
    kk = kb.float().cpu().numpy().astype(np.float64)[0, 0, 0]
    lse_exp = np.float64(np.float32(0.088388346)) * (qq @ kk) + np.log(Nk)
    assert np.max(np.abs(lse.cpu().numpy() - lse_exp)) <= 1e-3
    # One-hot selection: Q_i = e_{t(i)}, K_j = 64 e_j (Nk = d), scale 1 -> logit 64.
    t = r.integers(0, d, size=Nq)
    q1 = np.zeros((1, 1, Nq, d))
    q1[0, 0, np.arange(Nq), t] = 1.0
    k1 = (64.0 * np.eye(d))[None, None]
    v1 = r.standard_normal((1, 1, d, d))
    say("case structured one-hot")
    o, lse = fa.forward(_bf16_dev(q1), _bf16_dev(k1), _bf16_dev(v1), scale=1.0)
    torch.cuda.synchronize()
    v1b = synth.bf16_bits_to_f32(synth.bf16_bits(v1.astype(np.float32))).astype(np.float64)
    assert np.max(np.abs(o.float().cpu().numpy()[0, 0] - v1b[0, 0, t])) <= 1e-2
    assert np.max(np.abs(lse.cpu().numpy()[0, 0] - 64.0)) <= 1e-3
    say("case structured V = 1")
    o, _ = fa.forward(qb, _bf16_dev(r.standard_normal((1, 2, Nk, d))), _bf16_dev(np.ones((1, 2, Nk, d))),
                      causal=True)
    torch.cuda.synchronize()
    assert np.max(np.abs(o.float().cpu().numpy() - 1.0)) <= 8e-3


@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, False)])
def test_logit_ramps(d, causal):
    """Logits that rise, fall or stay flat across 32 key tiles (plus noise),
    spanning far more than the fp32 exponent range within one row: rising rows
    make the kernel move its exponent reference several times after rows have
    accumulated large sums, falling rows drive later tiles to underflow.
    Compared with the fp64 oracle on every row."""
    import torch
    fa = _fa()
    r = np.random.default_rng(11)
    Nq, Nk = 96, 2048
    # s_ij = a_i t_j + b_i u_j (scale 1): t is a ramp over the keys, u noise.
    t = np.linspace(-1.0, 1.0, Nk) * 90.0
    u = r.standard_normal(Nk) * 2.0
    k = np.zeros((1, 1, Nk, d))
    k[0, 0, :, 0] = t
    k[0, 0, :, 1] = u
    q = np.zeros((1, 1, Nq, d))
    q[0, 0, :, 0] = np.concatenate([np.linspace(0.2, 2.0, Nq // 3), -np.linspace(0.2, 2.0, Nq // 3),
                                    np.zeros(Nq - 2 * (Nq // 3))])
    q[0, 0, :, 1] = r.standard_normal(Nq)
    v = r.standard_normal((1, 1, Nk, d))
    qb, kb, vb = (_bf16_dev(x) for x in (q, k, v))
    say(f"case logit ramps d={d} causal={causal}")
    o, lse = fa.forward(qb, kb, vb, scale=1.0, causal=causal)
    torch.cuda.synchronize()
    to64 = lambda x: x.float().cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention(to64(qb), to64(kb), to64(vb), 1.0, causal)
    assert_close(errors(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref), what=f"ramps d={d} causal={causal}")


def test_gqa_equals_repeated_kv():
    import torch
    fa = _fa()
    w = synth.Workload("gqa", 2, 8, 2, 256, 320, 128, causal=True)
    q, k, v = device_inputs(w)
    say("case GQA vs repeated-KV MHA")
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(),
                        causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic():
    import torch
    fa = _fa()
    w = W["batched_prefill_b4h16_n2048_causal"]
    q, k, v = device_inputs(w)
    say("case determinism")
    a = fa.forward(q, k, v, causal=True)
    b = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_and_degenerate():
    import torch
    fa = _fa()
    dev = "cuda"
    q = torch.randn(1, 2, 5, 128, device=dev).to(torch.bfloat16)
    k0 = torch.empty(1, 2, 0, 128, device=dev, dtype=torch.bfloat16)
    say("case Nk = 0")
    o, lse = fa.forward(q, k0, k0.clone())
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    say("case Nq = 0 and B = 0")
    qe = torch.empty(1, 2, 0, 128, device=dev, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 7, 128, device=dev).to(torch.bfloat16)
    o, lse = fa.forward(qe, k, k)
    ob, lb = fa.forward(torch.empty(0, 2, 5, 128, device=dev, dtype=torch.bfloat16),
                        torch.empty(0, 2, 7, 128, device=dev, dtype=torch.bfloat16),
                        torch.empty(0, 2, 7, 128, device=dev, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert o.numel() == 0 and ob.numel() == 0
    say("case decode Nk = 0")
    o, lse = fa.decode(q[:, :, :1].contiguous(), k0, k0.clone(), 4)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_argument_errors_on_device():
    import torch
    fa = _fa()
    q = torch.randn(1, 1, 8, 128, device="cuda").to(torch.bfloat16)
    with pytest.raises(TypeError):
        fa.forward(q.float(), q.float(), q.float())
    buf = torch.zeros(1 * 1 * 8 * 128 + 8, device="cuda", dtype=torch.bfloat16)
    mis = buf[1:1 + 8 * 128].view(1, 1, 8, 128)  # 2-byte offset: not 16-byte aligned
    with pytest.raises(fa.FaError) as ei:
        fa.forward(mis, q, q)
    assert ei.value.status == 4
    with pytest.raises(fa.FaError) as ei:
        fa.forward(q, q, q, scale=-1.0)
    assert ei.value.status == 7
    small = fa.workspace_for(q[:, :, :1].contiguous(), 2)[:16]
    with pytest.raises(fa.FaError) as ei:
        fa.decode(q[:, :, :1].contiguous(), q, q, 2, workspace=small)
    assert ei.value.status == 5
