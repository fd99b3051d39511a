"""MI355X (gfx950) exact attention forward: Python binding of libfa.so.

The binding only marshals arguments: every step of the computation runs in the
library's HIP kernels. torch supplies device memory and streams. If the library
is not built, loading it raises; there is no fallback path.

Entry points with the C names (tensors in, status checked, nothing returned):
    fa_fwd, fa_fwd_fp32, fa_fwd_fp8, fa_bwd, fa_bwd_workspace_bytes, fa_fwd_splitkv, fa_fwd_splitkv_noalloc,
    fa_fwd_splitkv_paged, fa_combine, fa_splitkv_workspace_bytes, fa_status_str
Convenience wrappers that allocate the outputs:
    forward(q, k, v, causal=False, scale=None)            -> (o, lse)
    forward_fp32(q, k, v, causal=False, scale=None)       -> (o, lse)
    forward_fp8(q8, k8, v8, descale, causal=False, scale=None) -> (o, lse)
    backward(q, k, v, o, lse, dout, causal=False, scale=None) -> (dq, dk, dv)
    decode(q, k, v, num_splits, causal=False, scale=None, workspace=None) -> (o, lse)
    decode_paged(q, k_cache, v_cache, block_table, seq_lens, num_splits, ...) -> (o, lse)
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_ALIGN",
                5: "FA_ERR_WORKSPACE", 6: "FA_ERR_LAUNCH", 7: "FA_ERR_ARG"}

# Exported symbols and their C signatures (mirrors include/fa.h).
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_layout": (_I, [_I, _I, _I, _I, _I]),
    "fa_fwd_fp32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _F, _F, _F, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]),
    "fa_splitkv_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "fa_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "fa_fwd_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_fwd_splitkv_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S,
                                  _P]),
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_default_scale": (_F, [_I]),
    "fa_build_hash": (ctypes.c_char_p, []),
}

_lib = None
# The library must have been built from this source tree (fa_build_hash).
VERIFY_BUILD = True


class FaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {fa_status_str(status)}")


class StaleLibraryError(RuntimeError):
    """libfa.so was built from sources other than the ones in this tree."""


def lib():
    """Load libfa.so (raises if it has not been built, or was built from other sources)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_17_amd.build`")
        # torch ships its own HIP runtime under the same soname
        # (libamdhip64.so.7). Loaded first, it satisfies the library's
        # dependency; loaded after the library, it would be a second runtime
        # in the process, and kernels launched through the system one on
        # memory that torch's allocated fail to launch.
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if VERIFY_BUILD:
            from .srchash import source_hash
            built, tree = handle.fa_build_hash().decode(), source_hash()
            if built != tree:
                raise StaleLibraryError(f"{LIB_PATH} was built from sources {built}, the tree holds {tree}: "
                                        "rebuild it with `python -m exact_io_aware_17_amd.build`")
        _lib = handle
    return _lib


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def _check(fn, status):
    if status != FA_OK:
        raise FaError(fn, status)


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _dims(q, k, v, dtype):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("q/k/v shapes disagree")
    del torch
    return B, Hq, Hkv, Nq, Nk, d


def _default_scale(d, scale):
    """scale=None is argument defaulting: the library's own default for head size d."""
    return float(lib().fa_default_scale(int(d))) if scale is None else float(scale)


def _same_device(q, **tensors):
    """Every tensor argument must live on q's GPU: the C ABI cannot tell a host
    pointer from a device pointer, so a CPU tensor is refused here."""
    for name, t in tensors.items():
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, got {t.device}")


def _out_check(o, lse, q, odtype):
    import torch
    _same_device(q, o=o, lse=lse)
    if o.dtype != odtype or tuple(o.shape) != tuple(q.shape) or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")


# fa_fwd's work layouts (FA_LAYOUT_* in fa.h).
LAYOUT_NAMES = {0: "kv_parity", 1: "kv_parity_paired", 2: "rows", 3: "rows_paired", 4: "wide_one_group",
                5: "wide_two_groups"}


def fa_fwd_layout(B, Hq, Nq, d, causal) -> str:
    """Name of the work layout fa_fwd uses for this shape."""
    return LAYOUT_NAMES.get(int(lib().fa_fwd_layout(B, Hq, Nq, d, int(bool(causal)))), "unsupported")


def fa_fwd(q, k, v, o, lse, scale=None, causal=False, stream=None):
    """bf16 forward into caller-provided o (bf16, like q) and lse (fp32 [B,Hq,Nq])."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.bfloat16)
    _out_check(o, lse, q, torch.bfloat16)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                      _default_scale(d, scale), int(bool(causal)), _stream(stream))
    _check("fa_fwd", st)


def fa_fwd_fp32(q, k, v, o, lse, scale=None, causal=False, stream=None):
    import torch
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.float32)
    _out_check(o, lse, q, torch.float32)
    st = lib().fa_fwd_fp32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                           _default_scale(d, scale), int(bool(causal)), _stream(stream))
    _check("fa_fwd_fp32", st)


def fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits) -> int:
    return int(lib().fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, num_splits, workspace, scale=None, causal=False, stream=None):
    """Split-KV forward; `workspace` is a device tensor of at least
    fa_splitkv_workspace_bytes(...) bytes."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.bfloat16)
    _out_check(o, lse, q, torch.bfloat16)
    _same_device(q, workspace=workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                              _default_scale(d, scale), int(bool(causal)), int(num_splits), _ptr(workspace),
                              nbytes, _stream(stream))
    _check("fa_fwd_splitkv", st)


# Size of the scratch fa_fwd_splitkv_noalloc uses (FA_NOALLOC_SCRATCH_BYTES in fa.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, num_splits, scale=None, causal=False, stream=None):
    """Split-KV forward with the library's own fixed scratch instead of a
    workspace (for callers that cannot allocate); o, lse are the caller's."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.bfloat16)
    _out_check(o, lse, q, torch.bfloat16)
    st = lib().fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                      _default_scale(d, scale), int(bool(causal)), int(num_splits),
                                      _stream(stream))
    _check("fa_fwd_splitkv_noalloc", st)


def fa_fwd_splitkv_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, num_splits, workspace, scale=None,
                         causal=False, stream=None):
    """Split-KV forward over a paged cache: k_cache / v_cache bf16 [num_pages, Hkv, page_size, d],
    block_table int32 [B, max_pages], seq_lens int32 [B] (all on the GPU)."""
    import torch
    if q.dtype != torch.bfloat16 or q.dim() != 4 or not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError("q must be a contiguous bf16 [B, Hq, Nq, d] GPU tensor")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 [num_pages, Hkv, page_size, d] tensor on q's device")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes disagree")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_cache.shape
    if dk != d or block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("k_cache / block_table / seq_lens shapes disagree with q")
    _out_check(o, lse, q, torch.bfloat16)
    _same_device(q, workspace=workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa_fwd_splitkv_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, d, num_pages, page_size,
                                    block_table.shape[1], _default_scale(d, scale), int(bool(causal)),
                                    int(num_splits), _ptr(workspace), nbytes, _stream(stream))
    _check("fa_fwd_splitkv_paged", st)


def fa_combine(o_part, lse_part, o, lse, stream=None):
    """Merge o_part [B,Hq,S,Nq,d] fp32 / lse_part [B,Hq,S,Nq] fp32 into o (bf16) and lse."""
    import torch
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if o_part.dim() != 5 or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("o_part must be a contiguous [B, Hq, S, Nq, d] tensor")
    B, Hq, S, Nq, d = o_part.shape
    if tuple(lse_part.shape) != (B, Hq, S, Nq):
        raise ValueError("lse_part must be [B, Hq, S, Nq]")
    if o.dtype != torch.bfloat16 or tuple(o.shape) != (B, Hq, Nq, d) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o must be bf16 [B, Hq, Nq, d] and lse [B, Hq, Nq]")
    if lse.dtype != torch.float32 or not o.is_contiguous() or not lse.is_contiguous():
        raise ValueError("o and lse must be contiguous; lse float32")
    if o_part.device.type != "cuda":
        raise ValueError("o_part must be on the GPU")
    _same_device(o_part, lse_part=lse_part, o=o, lse=lse)
    st = lib().fa_combine(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), B, Hq, Nq, d, S, _stream(stream))
    _check("fa_combine", st)


def _fp8_view(t, name):
    """E4M3 tensors travel as uint8 bytes; torch's float8_e4m3fn is accepted too."""
    import torch
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 E4M3 codes or float8_e4m3fn, got {t.dtype}")
    return t


def fa_fwd_fp8(q, k, v, o, lse, descale, scale=None, causal=False, stream=None):
    """fp8 (E4M3, per-tensor descale) forward into caller-provided o (bf16
    [B,Hq,Nq,d]) and lse (fp32 [B,Hq,Nq]); descale = (q, k, v) factors."""
    import torch
    q, k, v = _fp8_view(q, "q"), _fp8_view(k, "k"), _fp8_view(v, "v")
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.uint8)
    _out_check(o, lse, q, torch.bfloat16)
    qd, kd, vd = (float(x) for x in descale)
    st = lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), qd, kd, vd, _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                          _default_scale(d, scale), int(bool(causal)), _stream(stream))
    _check("fa_fwd_fp8", st)


def forward_fp8(q, k, v, descale, causal=False, scale=None, stream=None):
    import torch
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, o, lse, descale, scale=scale, causal=causal, stream=stream)
    return o, lse


def fa_bwd_workspace_bytes(B, Hq, Nq, d) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, Hq, Nq, d))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale=None, causal=False, stream=None):
    """Backward into caller-provided dq (like q), dk, dv (like k) bf16 tensors."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v, torch.bfloat16)
    _same_device(q, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    for name, t, like in (("o", o, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(like.shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like {'q' if like is q else 'k'}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, Hq, Hkv, Nq, Nk, d, _default_scale(d, scale), int(bool(causal)), _ptr(workspace),
                      workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream))
    _check("fa_bwd", st)


def backward(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None, stream=None):
    import torch
    B, Hq, Nq, d = q.shape
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(B, Hq, Nq, d), 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale=scale, causal=causal, stream=stream)
    return dq, dk, dv


def forward(q, k, v, causal=False, scale=None, stream=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, stream=stream)
    return o, lse


def forward_fp32(q, k, v, causal=False, scale=None, stream=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa_fwd_fp32(q, k, v, o, lse, scale=scale, causal=causal, stream=stream)
    return o, lse


def workspace_for(q, num_splits):
    """A device byte tensor large enough for fa_fwd_splitkv (256-byte aligned by torch's allocator)."""
    import torch
    B, Hq, Nq, d = q.shape
    n = fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def split_views(workspace, B, Hq, Nq, d, num_splits):
    """(o_part, lse_part) views of a split-KV workspace (the layout fa.h documents)."""
    import torch
    rows = B * Hq * num_splits * Nq
    ob = (rows * d * 4 + 255) // 256 * 256
    o_part = workspace[: rows * d * 4].view(torch.float32).view(B, Hq, num_splits, Nq, d)
    lse_part = workspace[ob: ob + rows * 4].view(torch.float32).view(B, Hq, num_splits, Nq)
    return o_part, lse_part


def decode(q, k, v, num_splits, causal=False, scale=None, workspace=None, stream=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, num_splits)
    fa_fwd_splitkv(q, k, v, o, lse, num_splits, workspace, scale=scale, causal=causal, stream=stream)
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, num_splits, causal=False, scale=None, workspace=None,
                 stream=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, num_splits)
    fa_fwd_splitkv_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, num_splits, workspace, scale=scale,
                         causal=causal, stream=stream)
    return o, lse
