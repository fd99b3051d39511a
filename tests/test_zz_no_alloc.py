"""fa_fwd_splitkv_noalloc (the split-KV decode without a caller workspace)
against fa_fwd_splitkv, through the C ABI: the same kernels run, so O and LSE
must agree bit for bit. Two calls in a row, the second smaller, so that the
second one runs over whatever the first left in the library's scratch."""
import numpy as np
import pytest

import synth
from gpu_helpers import device_inputs, say

pytestmark = pytest.mark.gpu


def _both(w, causal=False):
    import torch
    import exact_io_aware_17_amd as fa
    q, k, v = device_inputs(w)
    o_ref, l_ref = fa.decode(q, k, v, w.num_splits, causal=causal, scale=w.scale)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, w.num_splits, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def _assert_same(o, lse, o_ref, l_ref):
    import torch
    a = o.cpu().view(torch.int16).numpy()
    b = o_ref.cpu().view(torch.int16).numpy()
    assert np.array_equal(a, b), "O differs from fa_fwd_splitkv"
    la, lb = lse.cpu().numpy(), l_ref.cpu().numpy()
    assert np.array_equal(la.view(np.int32), lb.view(np.int32)), "LSE differs from fa_fwd_splitkv"


def test_noalloc_matches_workspace_path_twice():
    big = synth.WORKLOADS["gqa_decode_b64_hq32_hkv8_kv8192"]
    say(f"noalloc call 1: {big.name} (partials {big.B * big.Hq * big.num_splits * big.d * 4} bytes)")
    _assert_same(*_both(big))
    small = synth.Workload("noalloc_small", 2, 8, 2, 3, 1000, 128, num_splits=5)
    say("noalloc call 2: B2 Hq8 Hkv2 Nq3 Nk1000 S5 causal")
    _assert_same(*_both(small, causal=True))
    tiny = synth.Workload("noalloc_d64", 1, 4, 1, 1, 77, 64, num_splits=3)
    say("noalloc call 3: B1 Hq4 Hkv1 Nq1 Nk77 d64 S3")
    _assert_same(*_both(tiny))


def test_noalloc_rejects_oversize_and_enqueues_nothing():
    import torch
    import exact_io_aware_17_amd as fa
    w = synth.Workload("noalloc_big", 64, 32, 8, 2, 64, 128, num_splits=16)
    assert fa.fa_splitkv_workspace_bytes(w.B, w.Hq, w.Nq, w.d, w.num_splits) > fa.NOALLOC_SCRATCH_BYTES
    q, k, v = device_inputs(w)
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device=q.device)
    with pytest.raises(fa.FaError, match="WORKSPACE"):
        fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    assert not o.any() and not lse.any()
