"""The LDS-poisoning debug build (host only): compiled with FA_LDS_POISON, the
forward kernels (bf16 at every head size, fp8) store all-ones to each copy's LDS destination right before the
copy is issued; the regular build has no such stores."""
import os
import re
import subprocess

import pytest

from exact_io_aware_17_amd import build as B


SOURCES = ["fa_fwd.hip", "fa_fwd_wide.hip", "fa_fwd_fp8.hip"]


def _asm(src, extra):
    src = os.path.join(B.CSRC, src)
    r = subprocess.run([B.hipcc(), *B.HIP_FLAGS, *extra, "--cuda-device-only", "-S", src, "-o", "-"],
                       capture_output=True, text=True)
    if r.returncode:
        pytest.skip(f"hipcc could not compile: {r.stderr[:200]}")
    return r.stdout


def _poisoned_copies(asm):
    """Copies whose preceding instructions (after the previous copy) store
    16 bytes to LDS and wait for it."""
    lines = [ln.strip() for ln in asm.splitlines() if ln.strip() and not ln.strip().startswith(";")]
    n_copy, n_poisoned, since = 0, 0, []
    for ln in lines:
        if ln.startswith("global_load_lds_dwordx4"):
            n_copy += 1
            window = since[-8:]
            if any(x.startswith("ds_write_b128") for x in window) and any("lgkmcnt(0)" in x for x in window):
                n_poisoned += 1
            since = []
        else:
            since.append(ln)
    return n_copy, n_poisoned


@pytest.mark.parametrize("src", SOURCES)
def test_poison_build_stores_before_every_copy(src):
    n, p = _poisoned_copies(_asm(src, ["-DFA_LDS_POISON"]))
    assert n > 0 and p == n, (n, p)


@pytest.mark.parametrize("src", SOURCES)
def test_regular_build_has_no_poison_stores(src):
    n, p = _poisoned_copies(_asm(src, []))
    assert n > 0 and p == 0, (n, p)
