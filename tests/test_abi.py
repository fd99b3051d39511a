"""The C ABI on the host (no GPU): the library loads, exports every function
include/fa.h declares with the parameter count the binding assumes, and rejects
bad arguments with the documented status before touching the GPU."""
import ctypes
import math
import os
import re

import pytest

import exact_io_aware_17_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000  # a 16-byte-aligned host address: never dereferenced, every call below fails validation


def _declarations():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"^\s*(fa_status|size_t|float|int|const char\s*\*)\s*(fa_\w+)\s*\(([^)]*)\)\s*;", text,
                         re.M | re.S):
        params = [p.strip() for p in m.group(3).split(",") if p.strip() and p.strip() != "void"]
        decls[m.group(2)] = (m.group(1), len(params))
    return decls


def test_header_declarations_found():
    d = _declarations()
    assert set(d) == {"fa_fwd", "fa_fwd_fp32", "fa_fwd_fp8", "fa_bwd", "fa_bwd_workspace_bytes",
                      "fa_splitkv_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
                      "fa_fwd_splitkv_paged", "fa_combine", "fa_status_str", "fa_default_scale",
                      "fa_build_hash", "fa_fwd_layout"}


def test_library_exports_every_declared_symbol():
    lib = fa.lib()
    for name, (_, nparams) in _declarations().items():
        assert hasattr(lib, name), name
        assert name in fa.SIGNATURES, name
        assert len(fa.SIGNATURES[name][1]) == nparams, name


def test_status_strings():
    for code, name in fa.STATUS_NAMES.items():
        assert fa.fa_status_str(code).startswith(name)
    assert "unknown" in fa.fa_status_str(99)


def _fwd(entry="fa_fwd", q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=16, Nk=16, d=128, scale=0.1, causal=0):
    return getattr(fa.lib(), entry)(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, None)


def test_forward_layouts():
    """fa_fwd's layout follows the grid size: 256-row blocks (row groups)
    once they fill the 256 CUs, 128-row KV-parity blocks below that, causal
    pairs of blocks when a head has at least two; head sizes 192/256 have
    their own kernel."""
    L = fa.fa_fwd_layout
    assert L(1, 8, 4096, 128, False) == "kv_parity"  # the pages' shape: 128 blocks of 256 rows
    assert L(4, 16, 2048, 128, False) == "rows"  # 512 blocks
    assert L(4, 16, 2048, 128, True) == "rows_paired"  # 4 x 16 x 4 pairs = 256
    assert L(1, 32, 16384, 128, True) == "rows_paired"
    assert L(1, 16, 2048, 128, True) == "kv_parity_paired"  # 64 pairs of 256-row blocks: too few
    assert L(1, 1, 256, 64, False) == "kv_parity"
    assert L(256, 1, 256, 64, False) == "rows"
    assert L(1, 2, 384, 128, True) == "kv_parity_paired"
    assert L(1, 2, 100, 128, True) == "kv_parity"  # one block per head: nothing to pair
    assert L(1, 8, 4096, 256, False) == "wide_two_groups"
    assert L(4, 16, 2048, 192, True) == "wide_one_group"
    assert L(1, 8, 4096, 96, False) == "unsupported"


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_fp32"])
def test_forward_argument_checks(entry):
    f = lambda **kw: _fwd(entry, **kw)  # noqa: E731
    for name in ("q", "k", "v", "o", "lse"):
        assert f(**{name: None}) == 1, name
        assert f(**{name: P + 2}) == 4, name
        assert f(**{name: P + 8}) == 4, name
    assert f(Hq=3, Hkv=2) == 2
    assert f(Hkv=0) == 2
    assert f(B=-1) == 2
    assert f(Nq=-5) == 2
    assert f(Nk=-1) == 2
    assert f(B=1 << 30, Hq=1 << 20, Hkv=1 << 20) == 2
    assert f(d=96) == 3
    assert f(d=512) == 3
    if entry == "fa_fwd_fp32":
        assert f(d=256) == 3  # head sizes 192 and 256: bf16 prefill only
        assert f(d=192) == 3
    assert f(d=160) == 3
    for s in (0.0, -0.5, math.inf, math.nan):
        assert f(scale=s) == 7, s
    assert f(causal=2) == 7
    assert f(causal=-1) == 7


def _fwd8(q=P, k=P, v=P, o=P, lse=P, ds=(0.01, 0.01, 0.01), B=1, Hq=2, Hkv=1, Nq=16, Nk=16, d=128, scale=0.1,
          causal=0):
    return fa.lib().fa_fwd_fp8(q, k, v, ds[0], ds[1], ds[2], o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, None)


def test_fp8_argument_checks():
    """Every rejected call returns before anything is launched (no GPU needed)."""
    for name in ("q", "k", "v", "o", "lse"):
        assert _fwd8(**{name: None}) == 1, name
        assert _fwd8(**{name: P + 8}) == 4, name
    assert _fwd8(Hq=3, Hkv=2) == 2
    assert _fwd8(B=-1) == 2
    assert _fwd8(d=64) == 3
    assert _fwd8(d=96) == 3
    for s in (0.0, -0.5, math.inf, math.nan):
        assert _fwd8(scale=s) == 7, s
    for ds in ((0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, math.nan), (1.0, math.inf, 1.0),
               (1e-30, 1e-30, 1.0), (1e30, 1e30, 1.0)):
        assert _fwd8(ds=ds) == 7, ds
    assert _fwd8(causal=2) == 7
    # Nothing to compute: accepted without a launch.
    assert _fwd8(q=None, o=None, lse=None, B=0, k=None, v=None) == 0


def test_bwd_workspace_and_argument_checks():
    """Host-side checks of fa_bwd; every rejected call returns before a launch."""
    lib = fa.lib()
    assert lib.fa_bwd_workspace_bytes(2, 3, 5, 128) == 256  # D of 30 rows, 120 bytes rounded up to 256
    assert lib.fa_bwd_workspace_bytes(1, 2, 100, 64) == 1024  # 800 bytes rounded up
    assert lib.fa_bwd_workspace_bytes(1, 1, 0, 64) == 0 + 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 4, 96) == 0
    assert lib.fa_bwd_workspace_bytes(-1, 1, 4, 64) == 0

    def f(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Nq=16, Nk=16, d=128, scale=0.1,
          causal=0, ws=P, wsb=1 << 20):
        return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, ws, wsb, None)
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert f(**{name: None}) == 1, name
        assert f(**{name: P + 8}) == 4, name
    assert f(ws=None) == 5
    assert f(wsb=100) == 5
    assert f(ws=P + 16) == 4
    assert f(d=256) == 3
    assert f(d=96) == 3
    assert f(Hq=3, Hkv=2) == 2
    assert f(scale=0.0) == 7
    assert f(causal=3) == 7
    assert f(B=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, ws=None) == 0


def test_empty_tensors_may_be_null_but_shapes_still_checked():
    # An empty K/V (Nk == 0) with NULL k, v is valid, so only check the cases
    # that still fail before any launch.
    assert _fwd(k=None, v=None, Nk=0, d=96) == 3
    assert _fwd(q=None, o=None, lse=None, Nq=0, Hq=3, Hkv=2) == 2


def test_workspace_bytes():
    ws = fa.fa_splitkv_workspace_bytes
    rows = 64 * 32 * 16 * 1
    o_bytes = (rows * 128 * 4 + 255) // 256 * 256
    assert ws(64, 32, 1, 128, 16) == o_bytes + (rows * 4 + 255) // 256 * 256
    assert ws(1, 1, 1, 64, 1) == 256 + 256
    assert ws(0, 4, 1, 128, 4) == 0 + 0
    assert ws(1, 1, 1, 96, 4) == 0
    assert ws(1, 1, 1, 128, 0) == 0
    assert ws(1, 1, 1, 128, 1025) == 0
    assert ws(-1, 1, 1, 128, 2) == 0


def _split(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nq=1, Nk=100, d=128, scale=0.1, causal=0, S=4,
           ws=0x100000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = fa.fa_splitkv_workspace_bytes(B, Hq, Nq, d, S)
    return fa.lib().fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, S, ws, ws_bytes, None)


def test_splitkv_argument_checks():
    assert _split(S=0) == 7
    assert _split(S=1025) == 7
    assert _split(ws=None) == 5
    assert _split(ws_bytes=100) == 5
    assert _split(ws=0x100000 + 16) == 4
    assert _split(q=None) == 1
    assert _split(Hq=7) == 2
    assert _split(d=80) == 3
    assert _split(scale=-1.0) == 7
    assert _split(B=70000) == 3  # grid z limit


def _noalloc(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nq=1, Nk=100, d=128, scale=0.1, causal=0, S=4):
    return fa.lib().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, S, None)


def test_noalloc_argument_checks():
    """Every rejection happens on the host, before the scratch is looked up."""
    assert _noalloc(S=0) == 7
    assert _noalloc(S=1025) == 7
    assert _noalloc(q=None) == 1
    assert _noalloc(o=P + 8) == 4
    assert _noalloc(Hq=7) == 2
    assert _noalloc(d=80) == 3
    assert _noalloc(d=256) == 3
    assert _noalloc(scale=math.inf) == 7
    # Partials beyond the fixed scratch: FA_ERR_WORKSPACE.
    big = dict(B=64, Hq=32, Hkv=8, Nq=2, Nk=8192, S=16)
    assert fa.fa_splitkv_workspace_bytes(64, 32, 2, 128, 16) > fa.NOALLOC_SCRATCH_BYTES
    assert _noalloc(**big) == 5
    assert fa.fa_splitkv_workspace_bytes(64, 32, 1, 128, 16) <= fa.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m, "FA_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES


def _paged(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nq=1, d=128, num_pages=64, page=16,
           max_pages=8, scale=0.1, causal=0, S=4, ws=0x100000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = fa.fa_splitkv_workspace_bytes(B, Hq, Nq, d, S)
    return fa.lib().fa_fwd_splitkv_paged(q, kc, vc, bt, sl, o, lse, B, Hq, Hkv, Nq, d, num_pages, page, max_pages,
                                         scale, causal, S, ws, ws_bytes, None)


def test_paged_argument_checks():
    for page in (0, 8, 24, 1 << 17, -16):
        assert _paged(page=page) == 7, page
    assert _paged(num_pages=-1) == 2
    assert _paged(max_pages=-1) == 2
    assert _paged(max_pages=1 << 28, page=1 << 10) == 2
    assert _paged(q=None) == 1
    assert _paged(o=P + 4) == 4
    assert _paged(d=96) == 3
    assert _paged(Hq=7) == 2
    assert _paged(scale=0.0) == 7
    assert _paged(causal=3) == 7
    assert _paged(S=0) == 7
    assert _paged(sl=None) == 1
    assert _paged(bt=None) == 1
    assert _paged(kc=None) == 1
    assert _paged(num_pages=0) == 2
    assert _paged(kc=P + 8) == 4
    assert _paged(bt=P + 2) == 4
    assert _paged(sl=P + 1) == 4
    assert _paged(ws=None) == 5
    assert _paged(ws_bytes=64) == 5
    assert _paged(ws=0x100000 + 64) == 4
    assert _paged(B=70000) == 3


def test_combine_argument_checks():
    c = fa.lib().fa_combine
    assert c(P, P, P, P, 2, 4, 1, 128, 0, None) == 7
    assert c(None, P, P, P, 2, 4, 1, 128, 4, None) == 1
    assert c(P, P, P + 4, P, 2, 4, 1, 128, 4, None) == 4
    assert c(P, P, P, P, 2, 4, 1, 32, 4, None) == 3
    assert c(P, P, P, P, -2, 4, 1, 128, 4, None) == 2


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()


def test_product_path_does_not_import_oracle():
    """The package and its sources never reference the test oracle."""
    pkg = os.path.join(ROOT, "exact_io_aware_17_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "oracle/" not in text, fn


def test_loaded_library_matches_source_tree():
    """A libfa.so built from other sources is refused; the one loaded here was
    built from this tree."""
    from exact_io_aware_17_amd.srchash import source_hash
    assert fa.lib().fa_build_hash().decode() == source_hash()


def test_stale_library_is_refused(monkeypatch):
    import exact_io_aware_17_amd.srchash as sh
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(sh, "source_hash", lambda: "0123456789abcdef")
    with pytest.raises(fa.StaleLibraryError):
        fa.lib()
    monkeypatch.setattr(fa, "_lib", None)


def test_default_scale_is_the_pages_dim_power():
    for d in (64, 128, 256, 1, 7):
        assert fa.lib().fa_default_scale(d) == pytest.approx(d ** -0.5, rel=1e-7)
        assert fa._default_scale(d, None) == float(__import__("numpy").float32(1.0 / math.sqrt(d)))
    assert fa.lib().fa_default_scale(0) == 0.0


def test_binding_refuses_host_tensors_before_any_launch():
    """Outputs, workspaces and partials on the CPU are refused in Python: the C
    ABI cannot tell a host pointer from a device pointer."""
    import torch
    dev = torch.device("meta")  # stands in for a GPU tensor without needing one
    q = torch.empty(1, 2, 16, 128, dtype=torch.bfloat16, device=dev)
    lse_cpu = torch.empty(1, 2, 16, dtype=torch.float32)
    o_cpu = torch.empty(1, 2, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be on"):
        fa._out_check(o_cpu, torch.empty(1, 2, 16, dtype=torch.float32, device=dev), q, torch.bfloat16)
    with pytest.raises(ValueError, match="must be on"):
        fa._out_check(torch.empty_like(q), lse_cpu, q, torch.bfloat16)
    with pytest.raises(ValueError, match="must be on"):
        fa._same_device(q, workspace=torch.empty(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_combine(torch.empty(1, 2, 3, 16, 128), torch.empty(1, 2, 3, 16), o_cpu, lse_cpu)


def test_library_shares_torchs_hip_runtime():
    """Loading the library before torch has been imported must still leave a
    single HIP runtime in the process (torch's): with two, kernels launched
    through one on memory allocated by the other fail to launch. Run in a
    fresh interpreter so that nothing has imported torch yet."""
    import subprocess
    import sys
    code = (
        "import os, sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(fa.__file__)))!r})\n"
        "import exact_io_aware_17_amd as fa\n"
        "fa.VERIFY_BUILD = False\n"
        "fa.lib()\n"
        "import torch\n"
        "maps = {l.split()[-1] for l in open(f'/proc/{os.getpid()}/maps') if 'libamdhip64' in l}\n"
        "print(len(maps), sorted(maps))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    n = int(r.stdout.split()[0])
    assert n == 1, f"HIP runtimes mapped: {r.stdout.strip()}"
