"""Helpers shared by the GPU tests: seeded device inputs, sampled oracle rows,
error metrics. The oracle side only ever sees inputs drawn by ``synth``."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

O_TOL = 2e-2      # max |O - O_ref| for bf16 inputs with fp32 accumulation
LSE_TOL = 1e-3    # max |LSE - LSE_ref|
F32_TOL = 1e-5    # both, for the fp32 path


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(w: synth.Workload, bf16=True, device="cuda"):
    import torch
    if bf16:
        def get(t, shape):
            bits = synth.draw_bf16(w.seed, t, shape)
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        def get(t, shape):
            return torch.from_numpy(synth.draw(w.seed, t, shape)).to(device)
    return get(synth.TENSOR_Q, w.q_shape), get(synth.TENSOR_K, w.kv_shape), get(synth.TENSOR_V, w.kv_shape)


def oracle_full(w: synth.Workload, bf16=True):
    q, k, v = synth.inputs_f64(w, bf16=bf16)
    return oracle.attention(q, k, v, w.scale, w.causal)


def oracle_sample(w: synth.Workload, heads, rows, bf16=True):
    """Oracle O [len(heads), len(rows), d], LSE [len(heads), len(rows)] for the
    given (b, h) query heads and query rows, drawing only the slabs needed."""
    rows = np.asarray(rows)
    group = w.Hq // w.Hkv
    outs_o, outs_l = [], []
    for (b, h) in heads:
        g = h // group
        q, k, v = synth.inputs_f64(w, bf16=bf16, q_heads=[(b, h)], kv_heads=[(b, g)], q_rows=rows)
        o, l = oracle.attention(q[:, None], k[:, None], v[:, None], w.scale, w.causal, q_index=rows, nq=w.Nq)
        outs_o.append(o[0, 0])
        outs_l.append(l[0, 0])
    return np.stack(outs_o), np.stack(outs_l)


def errors(o, o_ref, lse, lse_ref):
    """max abs errors, and O error relative to max|O_ref| and in Frobenius norm.
    LSE = -inf must match exactly."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "rows without keys differ"
    fin = np.isfinite(lse_ref)
    e_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    e_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    scale = float(np.max(np.abs(o_ref))) if o.size else 1.0
    fro = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30)) if o.size else 0.0
    return {"o_max": e_o, "lse_max": e_l, "o_rel_max": e_o / max(scale, 1e-30), "o_rel_fro": fro,
            "nan": bool(np.isnan(o).any() or np.isnan(lse).any())}


# Relative Frobenius error of O for bf16 inputs. Rounding P to bf16 for P.V and
# O to bf16 each contribute about 2^-9/sqrt(3) ~ 1.1e-3 (measured 2-2.5e-3);
# one 64-key tile dropped or read stale at Nk = 8192 moves O by about
# sqrt(64 / 8192) ~ 9e-2 of its norm, far above this bound, while the absolute
# O bound (2e-2) is about one standard deviation of |O| there.
O_FRO_TOL = 1e-2


def assert_close(err, o_tol=O_TOL, lse_tol=LSE_TOL, what="", o_fro_tol=O_FRO_TOL):
    say(f"  {what}: {err}")
    assert not err["nan"], f"{what}: NaN in output"
    assert err["o_max"] <= o_tol, f"{what}: max|O-O_ref| = {err['o_max']:.3e} > {o_tol}"
    assert err["lse_max"] <= lse_tol, f"{what}: max|LSE-LSE_ref| = {err['lse_max']:.3e} > {lse_tol}"
    assert err["o_rel_fro"] <= o_fro_tol, f"{what}: ||O-O_ref||/||O_ref|| = {err['o_rel_fro']:.3e} > {o_fro_tol}"


def sample_rows(nq, n_random=24, seed=0, tile=128):
    """Rows at tile edges, the ends, and a few random ones."""
    r = np.random.default_rng(seed)
    edges = [0, 1, 31, 32, 63, 64, tile - 1, tile, nq // 2, nq - tile, nq - 33, nq - 2, nq - 1]
    rows = set(x for x in edges if 0 <= x < nq)
    rows.update(r.integers(0, nq, size=min(n_random, nq)).tolist())
    return np.array(sorted(rows))


def _pages(x, page, mp):
    """[B, Hkv, Nk, d] -> [B * mp, Hkv, page, d], logical page j of sequence b at row b * mp + j."""
    B, Hkv, Nk, d = x.shape
    return x.reshape(B, Hkv, mp, page, d).transpose(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page, d)


def paged_numpy(k, v, page, seed, spare=5, filler=3.0):
    """Page caches [num_pages, Hkv, page, d] holding K/V [B, Hkv, Nk, d] under
    synth.page_table's permutation; unused slots hold `filler`."""
    B, Hkv, Nk, d = k.shape
    mp = -(-Nk // page)
    num_pages, table = synth.page_table(B, mp, seed, spare)
    pad = ((0, 0), (0, 0), (0, mp * page - Nk), (0, 0))
    out = []
    for x in (k, v):
        cache = np.full((num_pages, Hkv, page, d), filler, dtype=x.dtype)
        cache[table.reshape(-1)] = _pages(np.pad(x, pad), page, mp)
        out.append(cache)
    return out[0], out[1], table


def paged_device(k, v, page, seed, spare=5, filler=3.0):
    """The same layout built on the GPU from device K/V tensors."""
    import torch
    B, Hkv, Nk, d = k.shape
    mp = -(-Nk // page)
    num_pages, table = synth.page_table(B, mp, seed, spare)
    idx = torch.from_numpy(table.reshape(-1).astype(np.int64)).to(k.device)
    out = []
    for x in (k, v):
        if mp * page != Nk:
            x = torch.nn.functional.pad(x, (0, 0, 0, mp * page - Nk))
        pages = x.reshape(B, Hkv, mp, page, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page, d)
        cache = torch.full((num_pages, Hkv, page, d), filler, dtype=x.dtype, device=x.device)
        cache[idx] = pages
        out.append(cache.contiguous())
    return out[0], out[1], torch.from_numpy(table).to(k.device)
