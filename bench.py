"""Benchmark of the attention forward hot path on one MI355X.

Default run (N=1): the pages' benchmark shape (B=1, H=8, Nq=4096, Nk=8192,
d=128, bf16, non-causal) through fa_fwd, W warm-up steps then exactly K timed
steps; one JSON line on stdout. The line also carries, each timed the same
way with its own roofline (HBM traffic from the committed counter summaries
when their source hash matches) and a bounded CPU-oracle baseline:
  - the other prefill workloads (single head 256^2 d64, batched B4 H16 2048^2
    with and without the causal mask, long causal B1 H32 16384^2);
  - the split-KV decode workload (B=64, Hq=32, Hkv=8, Nk=8192, 16 splits) and
    the same decode over a paged K/V cache (16-key pages in a random order);
  - the pages' shape with OCP E4M3 inputs (fa_fwd_fp8) and at head sizes 256
    and 192;
  - the backward pass (fa_bwd) on the pages' shape;
and the machine: ROCm version and the shader clock rocm-smi reports while the
pages' shape runs back to back.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
  python bench.py --only prefill [--workload NAME] | prefill_fp8 | prefill_d256 | backward | decode | decode_paged
                  --steps 3   (short runs under a profiler)
  python bench.py --copy-calib                       (plain copy of known size, for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PREFILL = "pages_shape_h8_q4096_kv8192"
PREFILL_FP8 = "pages_shape_fp8_h8_q4096_kv8192"
PREFILL_D256 = "pages_shape_d256_h8_q4096_kv8192"
PREFILL_D192 = "pages_shape_d192_h8_q4096_kv8192"
DECODE = "gqa_decode_b64_hq32_hkv8_kv8192"
# The other prefill workloads, each timed in the default line with its own
# roofline and CPU baseline (the first is launch-bound: 8 workgroups).
OTHER_PREFILL = ["single_head_n256_d64", "batched_prefill_b4h16_n2048", "batched_prefill_b4h16_n2048_causal",
                 "long_causal_h32_n16384"]
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_io_aware_17_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


FWD_SOURCES = ["fa_fwd.hip", "fa_common.h"]
FWD8_SOURCES = ["fa_fwd_fp8.hip", "fa_common.h"]
FWD256_SOURCES = ["fa_fwd_wide.hip", "fa_common.h"]
BWD_SOURCES = ["fa_bwd.hip", "fa_common.h"]
DEC_SOURCES = ["fa_splitkv.hip", "fa_common.h"]


def traffic_from_profile(name, sources):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken from other kernel sources."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_sha(sources):
        return None
    return float(b.group(1))


def device_inputs(w, device):
    import torch

    def get(t, shape):
        bits = synth.draw_bf16(w.seed, t, shape)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return get(synth.TENSOR_Q, w.q_shape), get(synth.TENSOR_K, w.kv_shape), get(synth.TENSOR_V, w.kv_shape)


def time_steps(step, steps, warmup, min_warm_s=0.0):
    """W untimed steps, then exactly K timed steps. Returns (wall seconds, mean
    step milliseconds from HIP events). One event pair brackets the K steps on
    the stream the kernels run on (the current torch stream, which the binding
    passes down), so the mean covers the launches and the gaps between them
    (about 0.1 us per launch here). An event pair around every step would put
    two marker packets between consecutive kernels: on this stack that adds
    about 6% to the step time and about 2% to each bracketed kernel."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The GPU clock ramps under sustained load; warm-up steps plus at least
    # min_warm_s of untimed work put the timed steps at the steady clock.
    t_end = time.perf_counter() + min_warm_s
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1) / steps
    return wall, ev_ms


def bench_prefill(w, steps, warmup, device, min_warm_s=0.2):
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = device_inputs(w, device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device)

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale=w.scale, causal=w.causal)
    wall, ev_ms = time_steps(step, steps, warmup, min_warm_s)
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ev_ms,
            "tflops": w.flops() / (wall / steps) / 1e12, "kernel_tflops": w.flops() / (ev_ms * 1e-3) / 1e12,
            "layout": fa.fa_fwd_layout(w.B, w.Hq, w.Nq, w.d, w.causal)}


def fwd_kernel_label(w, layout):
    """The kernel instance fa_fwd launches for workload w in `layout`."""
    if layout.startswith("wide"):
        return f"fwd_bf16_wide_kernel<{w.d}, {1 if layout == 'wide_one_group' else 2}>"
    paired = "true" if layout.endswith("paired") else "false"
    rows = "true" if layout.startswith("rows") else "false"
    return f"fwd_bf16_kernel<{w.d}, {paired}, {rows}>"


def bench_prefill_fp8(w, steps, warmup, device, min_warm_s=0.2):
    """fa_fwd_fp8 on E4M3 inputs (seeded draws / per-tensor descale)."""
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = (torch.from_numpy(synth.draw_e4m3(w.seed, t, s)).to(device)
               for t, s in ((synth.TENSOR_Q, w.q_shape), (synth.TENSOR_K, w.kv_shape), (synth.TENSOR_V, w.kv_shape)))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device)

    def step():
        fa.fa_fwd_fp8(q, k, v, o, lse, synth.FP8_DESCALE, scale=w.scale, causal=w.causal)
    wall, ev_ms = time_steps(step, steps, warmup, min_warm_s)
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ev_ms,
            "tflops": w.flops() / (wall / steps) / 1e12, "kernel_tflops": w.flops() / (ev_ms * 1e-3) / 1e12}


def bench_backward(w, steps, warmup, device, min_warm_s=0.2):
    """fa_bwd (D, then the dK/dV and dQ kernels) with O and LSE from one fa_fwd
    outside the timed steps; dO seeded like the inputs. FLOPs: the five
    products of the chain rule, 2.5 times the forward's (the dQ kernel computes
    S and dP a second time: 3.5 times the forward's MFMA work is executed)."""
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = device_inputs(w, device)
    bits = synth.draw_bf16(w.seed, synth.TENSOR_DO, w.q_shape)
    do = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(*w.q_shape), dtype=torch.uint8, device=device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=w.scale, causal=w.causal)
    wall, ev_ms = time_steps(step, steps, warmup, min_warm_s)
    fl = 2.5 * w.flops()
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ev_ms,
            "tflops": fl / (wall / steps) / 1e12, "kernel_tflops": fl / (ev_ms * 1e-3) / 1e12}


def bench_decode(w, steps, warmup, device, min_warm_s=0.2):
    """Each step reads a different copy of K/V (three copies rotate) so that no
    step finds its 2 GiB of K/V in the 256 MB last-level cache."""
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = device_inputs(w, device)
    copies = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device)
    ws = fa.workspace_for(q, w.num_splits)
    it = [0]

    def step():
        kk, vv = copies[it[0] % len(copies)]
        it[0] += 1
        fa.fa_fwd_splitkv(q, kk, vv, o, lse, w.num_splits, ws, scale=w.scale)
    wall, ev_ms = time_steps(step, steps, warmup, min_warm_s)
    nbytes = w.algorithmic_bytes()
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ev_ms,
            "gbs": nbytes / (wall / steps) / 1e9, "kernel_gbs": nbytes / (ev_ms * 1e-3) / 1e9}


PAGE = 16  # keys per page of the paged decode benchmark


def paged_caches(k, v, page, seed):
    """K/V [B, Hkv, Nk, d] laid out as page caches [num_pages, Hkv, page, d]
    in the seeded random page order of synth.page_table; returns
    (k_cache, v_cache, block_table int32 [B, max_pages])."""
    import torch
    B, Hkv, Nk, d = k.shape
    mp = -(-Nk // page)
    num_pages, table = synth.page_table(B, mp, seed)
    idx = torch.from_numpy(table.reshape(-1).astype("int64")).to(k.device)
    out = []
    for x in (k, v):
        if mp * page != Nk:
            x = torch.nn.functional.pad(x, (0, 0, 0, mp * page - Nk))
        pages = x.reshape(B, Hkv, mp, page, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page, d)
        cache = torch.empty((num_pages, Hkv, page, d), dtype=x.dtype, device=x.device)
        cache[idx] = pages
        out.append(cache)
    return out[0], out[1], torch.from_numpy(table).to(k.device)


def bench_decode_paged(w, steps, warmup, device, page=PAGE, min_warm_s=0.2):
    """The decode workload over paged K/V (16-key pages in a random order);
    three caches rotate so that no step reads cache-warm data."""
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = device_inputs(w, device)
    caches = [paged_caches(k, v, page, seed=w.seed + i) for i in range(3)]
    del k, v
    sl = torch.full((w.B,), w.Nk, dtype=torch.int32, device=device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device)
    ws = fa.workspace_for(q, w.num_splits)
    it = [0]

    def step():
        kc, vc, table = caches[it[0] % len(caches)]
        it[0] += 1
        fa.fa_fwd_splitkv_paged(q, kc, vc, table, sl, o, lse, w.num_splits, ws, scale=w.scale)
    wall, ev_ms = time_steps(step, steps, warmup, min_warm_s)
    nbytes = w.algorithmic_bytes() + caches[0][2].numel() * 4 + w.B * 4  # + block table and lengths
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "kernel_ms": ev_ms, "page": page,
            "gbs": nbytes / (wall / steps) / 1e9, "kernel_gbs": nbytes / (ev_ms * 1e-3) / 1e9}


def host_info():
    """CPU model, BLAS library and the threads it uses (for the CPU baselines)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas, "cores": threads}


def _visible_keys(w, rows):
    """Keys each query row sees (the bottom-right causal reading)."""
    rows = np.asarray(rows, dtype=np.int64)
    if not w.causal:
        return np.full(rows.shape, w.Nk, dtype=np.int64)
    return np.clip(rows + 1 + (w.Nk - w.Nq), 0, w.Nk)


def cpu_baseline(w, budget_s=15.0, row_block=1024, kind="attention"):
    """The fp64 oracle on the host over a bounded sample of the workload: (batch,
    head) slabs in order, each in blocks of query rows, until the budget is
    spent. Prefill reports TFLOP/s (the FLOPs of the rows done); decode reports
    GB/s (the algorithmic bytes of the slabs done, as for the GPU line).
    `kind` picks the oracle: "attention" (bf16 inputs), "fp8" (E4M3 inputs,
    decoded inside the timed call), "backward" (the gradients of a row block
    against all of its head's keys: dQ of those rows and their share of dK
    and dV; credited 2.5x the forward FLOPs, as the GPU line) or "paged"
    (one sequence at a time, its keys gathered from a page cache in a random
    page order)."""
    import oracle
    if kind == "paged":
        return _cpu_baseline_paged(w, budget_s)
    group = w.Hq // w.Hkv
    t_total, flops, rows_done, slabs = 0.0, 0.0, 0, 0
    for b in range(w.B):
        for h in range(w.Hq):
            for r0 in range(0, w.Nq, row_block):
                rows = np.arange(r0, min(w.Nq, r0 + row_block))
                if kind == "fp8":
                    q8 = synth.draw_e4m3(w.seed, synth.TENSOR_Q, w.q_shape, heads=[(b, h)], rows=rows)
                    k8 = synth.draw_e4m3(w.seed, synth.TENSOR_K, w.kv_shape, heads=[(b, h // group)])
                    v8 = synth.draw_e4m3(w.seed, synth.TENSOR_V, w.kv_shape, heads=[(b, h // group)])
                    t0 = time.perf_counter()
                    oracle.attention_fp8(q8[:, None], k8[:, None], v8[:, None], synth.FP8_DESCALE, w.scale,
                                         w.causal, q_index=rows, nq=w.Nq)
                elif kind == "backward":
                    q, k, v = synth.inputs_f64(w, q_heads=[(b, h)], kv_heads=[(b, h // group)], q_rows=rows)
                    do = synth.bf16_bits_to_f32(synth.draw_bf16(w.seed, synth.TENSOR_DO, w.q_shape,
                                                                heads=[(b, h)], rows=rows)).astype(np.float64)
                    if w.causal:
                        raise ValueError("the backward baseline samples row blocks of non-causal workloads")
                    t0 = time.perf_counter()
                    oracle.attention_backward_head(q[0], k[0], v[0], do[0], w.scale, False)
                else:
                    q, k, v = synth.inputs_f64(w, q_heads=[(b, h)], kv_heads=[(b, h // group)], q_rows=rows)
                    t0 = time.perf_counter()
                    oracle.attention(q[:, None], k[:, None], v[:, None], w.scale, w.causal, q_index=rows, nq=w.Nq)
                t_total += time.perf_counter() - t0
                flops += (2.5 if kind == "backward" else 1.0) * 4.0 * w.d * float(_visible_keys(w, rows).sum())
                rows_done += len(rows)
                if t_total >= budget_s:
                    break
            slabs += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    out = host_info()
    frac = rows_done / max(w.B * w.Hq * w.Nq, 1)
    what = {"attention": "fp64 numpy", "fp8": "E4M3 decode + fp64 numpy",
            "backward": "fp64 numpy gradients"}[kind]
    sample = (f"{rows_done} of {w.B * w.Hq * w.Nq} query rows ({slabs} (batch, head) slabs) of {w.name}, "
              f"{t_total:.1f} s of {what} on the host")
    if w.num_splits:
        return {"value": w.algorithmic_bytes() * frac / t_total / 1e9, "unit": "GB/s",
                "cores": out["cores"], "kind": "oracle", "sample": sample,
                "cpu_model": out["cpu_model"], "blas": out["blas"]}
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": out["cores"], "kind": "oracle",
            "sample": sample, "cpu_model": out["cpu_model"], "blas": out["blas"]}


def _cpu_baseline_paged(w, budget_s, page=PAGE):
    """cpu_baseline for the paged decode: per sequence, its K/V pages stored in
    a random page order, then the oracle's gather and attention (timed)."""
    import oracle
    t_total, seqs = 0.0, 0
    n_pages = -(-w.Nk // page)
    for b in range(w.B):
        q, k, v = synth.inputs_f64(w, q_heads=[(b, h) for h in range(w.Hq)],
                                   kv_heads=[(b, h) for h in range(w.Hkv)])
        _, table = synth.page_table(1, n_pages, w.seed + b)
        pad = n_pages * page - w.Nk
        kp = np.pad(k, ((0, 0), (0, pad), (0, 0))).reshape(w.Hkv, n_pages, page, w.d).transpose(1, 0, 2, 3)
        vp = np.pad(v, ((0, 0), (0, pad), (0, 0))).reshape(w.Hkv, n_pages, page, w.d).transpose(1, 0, 2, 3)
        k_cache = np.empty_like(kp)
        v_cache = np.empty_like(vp)
        k_cache[table[0]] = kp
        v_cache[table[0]] = vp
        t0 = time.perf_counter()
        oracle.paged_attention(q[None], k_cache, v_cache, table, np.array([w.Nk]), w.scale, w.causal)
        t_total += time.perf_counter() - t0
        seqs += 1
        if t_total >= budget_s:
            break
    out = host_info()
    nbytes = (w.algorithmic_bytes() + w.B * n_pages * 4 + w.B * 4) * seqs / w.B
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": out["cores"], "kind": "oracle",
            "sample": f"{seqs} of {w.B} sequences of {w.name}_paged{page} ({page}-key pages in a random order), "
                      f"{t_total:.1f} s of fp64 numpy on the host",
            "cpu_model": out["cpu_model"], "blas": out["blas"]}


def rocm_version():
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            continue
    return None


def _read_sclk_mhz():
    """Current shader clock(s) in MHz from rocm-smi (a child process)."""
    import subprocess
    for exe in ("rocm-smi", "/opt/rocm/bin/rocm-smi"):
        try:
            out = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=20).stdout
        except (OSError, subprocess.TimeoutExpired):
            continue
        try:
            data = json.loads(out)
        except ValueError:
            continue
        vals = []
        for card in data.values():
            if isinstance(card, dict):
                for key, val in card.items():
                    if "sclk" in key.lower() and "speed" in key.lower():
                        m = re.search(r"(\d+)\s*Mhz", str(val), re.I)
                        if m:
                            vals.append(int(m.group(1)))
        if vals:
            return vals
    return None


def sustained_sclk(step, seconds=2.0):
    """Shader clock while `step` runs back to back for `seconds`: rocm-smi is
    polled from a thread; returns the median, min and max MHz it reported."""
    import threading
    import torch
    readings, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            v = _read_sclk_mhz()
            if v is None:
                return
            readings.extend(v)

    th = threading.Thread(target=poll, daemon=True)
    t_end = time.perf_counter() + seconds
    for _ in range(20):
        step()
    torch.cuda.synchronize()
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    if not readings:
        return {"sclk_mhz": None, "how": "rocm-smi --showclocks gave no reading"}
    r = sorted(readings)
    return {"sclk_mhz": r[len(r) // 2], "sclk_mhz_min": r[0], "sclk_mhz_max": r[-1], "readings": len(r),
            "how": f"rocm-smi --showclocks polled while the pages' shape prefill ran back to back for {seconds} s"}


def copy_calib(device, nbytes=1 << 30, steps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes": nbytes, "steps": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all", action="store_true", help="(kept for old command lines; the other prefill "
                                                          "workloads are always timed)")
    ap.add_argument("--only", choices=["prefill", "prefill_fp8", "prefill_d256", "prefill_d192", "backward", "decode",
                                       "decode_paged"],
                    default=None)
    ap.add_argument("--workload", default=None, help="with --only prefill: the prefill workload (synth name)")
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    if args.copy_calib:
        copy_calib(device)
        return
    from __graft_entry__ import _ensure_built
    _ensure_built()

    wp = synth.WORKLOADS[PREFILL]
    wd = synth.WORKLOADS[DECODE]
    if args.only == "prefill":
        w = synth.WORKLOADS[args.workload] if args.workload else wp
        r = bench_prefill(w, args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": "prefill", "workload": w.name, **r}))
        return
    if args.only == "backward":
        r = bench_backward(wp, args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": "backward", **r}))
        return
    if args.only in ("prefill_d256", "prefill_d192"):
        name = PREFILL_D256 if args.only == "prefill_d256" else PREFILL_D192
        r = bench_prefill(synth.WORKLOADS[name], args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": args.only, **r}))
        return
    if args.only == "prefill_fp8":
        r = bench_prefill_fp8(synth.WORKLOADS[PREFILL_FP8], args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": "prefill_fp8", **r}))
        return
    if args.only == "decode":
        r = bench_decode(wd, args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": "decode", **r}))
        return
    if args.only == "decode_paged":
        r = bench_decode_paged(wd, args.steps, args.warmup, device, min_warm_s=0.0)
        print(json.dumps({"only": "decode_paged", **r}))
        return

    log(f"prefill {wp.name}: warmup {args.warmup}, steps {args.steps}")
    rp = bench_prefill(wp, args.steps, args.warmup, device)
    log(f"  {rp}")
    w8 = synth.WORKLOADS[PREFILL_FP8]
    log(f"prefill fp8 {w8.name}: warmup {args.warmup}, steps {args.steps}")
    r8 = bench_prefill_fp8(w8, args.steps, args.warmup, device)
    log(f"  {r8}")
    w256 = synth.WORKLOADS[PREFILL_D256]
    log(f"prefill d256 {w256.name}: warmup {args.warmup}, steps {args.steps}")
    r256 = bench_prefill(w256, args.steps, args.warmup, device)
    log(f"  {r256}")
    w192 = synth.WORKLOADS[PREFILL_D192]
    log(f"prefill d192 {w192.name}: warmup {args.warmup}, steps {args.steps}")
    r192 = bench_prefill(w192, args.steps, args.warmup, device)
    log(f"  {r192}")
    bsteps, bwarm = max(1, args.steps // 5), max(1, args.warmup // 5)
    log(f"backward {wp.name}: warmup {bwarm}, steps {bsteps}")
    rb = bench_backward(wp, bsteps, bwarm, device)
    log(f"  {rb}")
    log(f"decode {wd.name}: warmup {args.warmup}, steps {args.steps}")
    rd = bench_decode(wd, args.steps, args.warmup, device)
    log(f"  {rd}")
    log(f"paged decode {wd.name}, {PAGE}-key pages: warmup {args.warmup}, steps {args.steps}")
    rdp = bench_decode_paged(wd, args.steps, args.warmup, device)
    log(f"  {rdp}")
    others = {}
    for name in OTHER_PREFILL:
        w = synth.WORKLOADS[name]
        log(f"prefill {name}: warmup {args.warmup}, steps {args.steps}")
        r = bench_prefill(w, args.steps, args.warmup, device)
        log(f"  {r}")
        others[name] = {
            "workload": name, "B": w.B, "H": w.Hq, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
            "metric": "attention fwd TFLOPS (4*B*H*Nq*Nk*d per forward, halved under the causal mask)",
            "value": round(r["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(r["ms_per_step"], 5),
            "roofline": {"bound": "mfma", "achieved": round(r["kernel_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profile(f"fwd_bf16_{name}_traffic.md", FWD_SOURCES),
                         "kernel_ms": round(r["kernel_ms"], 5),
                         "kernel": fwd_kernel_label(w, r["layout"]), "layout": r["layout"]}}
    log("sustained shader clock ...")
    wsc = synth.WORKLOADS[PREFILL]
    import exact_io_aware_17_amd as fa
    q_, k_, v_ = device_inputs(wsc, device)
    o_, l_ = torch.empty_like(q_), torch.empty(q_.shape[:3], dtype=torch.float32, device=device)
    clock = sustained_sclk(lambda: fa.fa_fwd(q_, k_, v_, o_, l_, scale=wsc.scale))
    del q_, k_, v_, o_, l_
    log(f"  {clock}")

    fwd_traffic = traffic_from_profile("fwd_bf16_pages_shape_traffic.md", FWD_SOURCES)
    fwd8_traffic = traffic_from_profile("fwd_fp8_pages_shape_traffic.md", FWD8_SOURCES)
    fwd256_traffic = traffic_from_profile("fwd_bf16_d256_pages_shape_traffic.md", FWD256_SOURCES)
    bwd_traffic = traffic_from_profile("bwd_pages_shape_traffic.md", BWD_SOURCES)
    dec_traffic = traffic_from_profile("splitkv_decode_traffic.md", DEC_SOURCES)
    decp_traffic = traffic_from_profile("splitkv_paged_decode_traffic.md", DEC_SOURCES)
    line = {
        "metric": "attention fwd TFLOPS (4*B*H*Nq*Nk*d per forward) on the pages' shape; decode HBM GB/s",
        "value": round(rp["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rp["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wp.name, "B": wp.B, "H": wp.Hq, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d,
                   "causal": wp.causal, "pct_of_bf16_peak": round(100 * rp["tflops"] / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(rp["kernel_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(rp["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": fwd_traffic, "kernel_ms": round(rp["kernel_ms"], 5),
                     "kernel": fwd_kernel_label(wp, rp["layout"]), "layout": rp["layout"]},
        "prefill_fp8": {"workload": w8.name, "dtype": "fp8 e4m3 (per-tensor descale), bf16 out",
                        "metric": "attention fwd TFLOPS (4*B*H*Nq*Nk*d per forward)", "value": round(r8["tflops"], 2),
                        "unit": "TFLOP/s", "ms_per_step": round(r8["ms_per_step"], 5),
                        "roofline": {"bound": "mfma", "achieved": round(r8["kernel_tflops"], 2),
                                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(r8["kernel_tflops"] / PEAK_FP8_TFLOPS, 4), "traffic": fwd8_traffic,
                                     "kernel_ms": round(r8["kernel_ms"], 5), "kernel": "fwd_fp8_kernel"}},
        "prefill_d256": {"workload": w256.name, "dtype": "bf16", "d": 256,
                         "metric": "attention fwd TFLOPS (4*B*H*Nq*Nk*d per forward)",
                         "value": round(r256["tflops"], 2), "unit": "TFLOP/s",
                         "ms_per_step": round(r256["ms_per_step"], 5),
                         "roofline": {"bound": "mfma", "achieved": round(r256["kernel_tflops"], 2),
                                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(r256["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                                      "traffic": fwd256_traffic, "kernel_ms": round(r256["kernel_ms"], 5),
                                      "kernel": "fwd_bf16_wide_kernel<256, 2>"}},
        "prefill_d192": {"workload": w192.name, "dtype": "bf16", "d": 192,
                         "metric": "attention fwd TFLOPS (4*B*H*Nq*Nk*d per forward)",
                         "value": round(r192["tflops"], 2), "unit": "TFLOP/s",
                         "ms_per_step": round(r192["ms_per_step"], 5),
                         "roofline": {"bound": "mfma", "achieved": round(r192["kernel_tflops"], 2),
                                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(r192["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                                      "traffic": traffic_from_profile("fwd_bf16_d192_pages_shape_traffic.md",
                                                                      FWD256_SOURCES),
                                      "kernel_ms": round(r192["kernel_ms"], 5),
                                      "kernel": "fwd_bf16_wide_kernel<192, 2>"}},
        "backward": {"workload": wp.name, "dtype": "bf16",
                     "metric": "attention bwd TFLOPS (2.5 x 4*B*H*Nq*Nk*d: the five products)",
                     "value": round(rb["tflops"], 2), "unit": "TFLOP/s", "steps": bsteps, "warmup": bwarm,
                     "ms_per_step": round(rb["ms_per_step"], 5),
                     "roofline": {"bound": "mfma", "achieved": round(rb["kernel_tflops"], 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(rb["kernel_tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": bwd_traffic,
                                  "kernel_ms": round(rb["kernel_ms"], 5),
                                  "kernel": "bwd_prep_kernel<128> + bwd_dkdv_kernel<128> + bwd_dq_kernel<128>"}},
        "decode": {"workload": wd.name, "metric": "decode HBM GB/s (algorithmic bytes / step time)",
                   "value": round(rd["gbs"], 1), "unit": "GB/s", "ms_per_step": round(rd["ms_per_step"], 5),
                   "roofline": {"bound": "hbm", "achieved": round(rd["kernel_gbs"], 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(rd["kernel_gbs"] / PEAK_HBM_GBS, 4),
                                "traffic": dec_traffic, "kernel_ms": round(rd["kernel_ms"], 5),
                                "kernel": "splitkv_partial_kernel<128, false> + combine_kernel<128>"}},
        "decode_paged": {"workload": f"{wd.name}_paged{PAGE}", "page_size": PAGE,
                         "metric": "paged decode HBM GB/s (algorithmic bytes incl. block table / step time)",
                         "value": round(rdp["gbs"], 1), "unit": "GB/s", "ms_per_step": round(rdp["ms_per_step"], 5),
                         "roofline": {"bound": "hbm", "achieved": round(rdp["kernel_gbs"], 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(rdp["kernel_gbs"] / PEAK_HBM_GBS, 4), "traffic": decp_traffic,
                                      "kernel_ms": round(rdp["kernel_ms"], 5),
                                      "kernel": "splitkv_partial_kernel<128, true> + combine_kernel<128>"}},
    }
    line["other_prefill"] = others
    line["machine"] = {"rocm": rocm_version(), "gpu": torch.cuda.get_device_name(0), **clock,
                       "peak_note": "frac is against the published peaks (2.5 PFLOP/s dense bf16 at 2.4 GHz, "
                                    "5.0 fp8, 8 TB/s HBM)"}
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(wp, budget_s=8.0)
        log(f"  {line['cpu_baseline']}")
        for name in OTHER_PREFILL:
            others[name]["cpu_baseline"] = cpu_baseline(synth.WORKLOADS[name], budget_s=3.0)
            log(f"  {name}: {others[name]['cpu_baseline']}")
        line["decode"]["cpu_baseline"] = cpu_baseline(wd, budget_s=3.0)
        log(f"  decode: {line['decode']['cpu_baseline']}")
        for key, wl, kind in (("prefill_fp8", w8, "fp8"), ("prefill_d256", w256, "attention"),
                              ("prefill_d192", w192, "attention"), ("backward", wp, "backward"),
                              ("decode_paged", wd, "paged")):
            line[key]["cpu_baseline"] = cpu_baseline(wl, budget_s=2.0, kind=kind)
            log(f"  {key}: {line[key]['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
