"""Build the gfx950 attention library (libfa.so) in-tree with hipcc.

Usage: python -m exact_io_aware_17_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

try:
    from .srchash import source_hash
except ImportError:  # run as a script
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from exact_io_aware_17_amd.srchash import source_hash

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libfa.so")
# Debug build: every tile copy first fills its LDS destination with NaN
# (FA_LDS_POISON), so that a read racing a copy shows up as NaN in O.
POISON_BUILD_DIR = os.path.join(HERE, "_build_poison")
POISON_LIB_PATH = os.path.join(HERE, "libfa_poison.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_wide.hip", "fa_fwd_fp8.hip", "fa_fp32.hip", "fa_splitkv.hip", "fa_bwd.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags=None, poison: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libfa.so (or, with
    poison=True, the LDS-poisoning debug library libfa_poison.so); returns its
    path. The hash of the sources is compiled in (fa_build_hash)."""
    cc = hipcc()
    build_dir, lib_path = (POISON_BUILD_DIR, POISON_LIB_PATH) if poison else (BUILD_DIR, LIB_PATH)
    os.makedirs(build_dir, exist_ok=True)
    flags = HIP_FLAGS + [f'-DFA_SOURCE_HASH="{source_hash()}"'] + (["-DFA_LDS_POISON"] if poison else [])
    flags += list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib_path + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
    print(build(verbose="-v" in sys.argv[1:], poison=True))
