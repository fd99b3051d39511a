"""Seeded synthetic inputs for the attention forward workloads.

This module is shared by the test-side oracle and by the GPU path's callers
(tests, benchmark, smoke check). It holds no part of the attention arithmetic:
only random draws, the fp32 -> bf16 storage encoding of those draws, and the
named workload shapes.

Recipe (stated once, used everywhere):

* Every tensor is a set of independent (batch, head) slabs of shape (N, d).
  Slab (b, h) of tensor ``t`` (0 = Q, 1 = K, 2 = V, 3 = dO) is drawn as
  ``standard_normal((N, d), float32)`` from a PCG64 generator seeded with
  ``SeedSequence([seed, t, b, h])``.  Slabs can therefore be drawn one at a
  time (for sampled checks of large workloads) or in parallel threads, and the
  values never depend on how many slabs are drawn together.
* The bf16 inputs are those fp32 draws rounded to nearest-even on the bit
  pattern: ``(u + 0x7FFF + ((u >> 16) & 1)) >> 16`` (finite values only; a
  normal draw is always finite).  The fp32 debug path uses the unrounded draws.
* Q has shape [B, Hq, Nq, d]; K and V have shape [B, Hkv, Nk, d]; all are
  contiguous row-major with d innermost.
* The fp8 inputs are the same fp32 draws divided by a fixed per-tensor
  descale factor (``FP8_DESCALE``: 6.75/448 for Q, 6.5/448 for K, 6.25/448
  for V, so a draw of about 6.5 standard deviations maps to the largest
  finite value 448) and encoded as OCP E4M3 (1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals, no infinities) with round to nearest,
  ties to even; the rare magnitudes beyond 448 saturate to +-448.  The value a
  byte stands for is (its E4M3 value) * descale.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
TENSOR_DO = 3  # the output gradient dO of the backward pass


@dataclass(frozen=True)
class Workload:
    """One attention-forward workload: shapes, mask and (for decode) splits."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool = False
    num_splits: int = 0  # > 0: split-KV decode with this many key chunks
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32, the value handed to the library."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def q_shape(self):
        return (self.B, self.Hq, self.Nq, self.d)

    @property
    def kv_shape(self):
        return (self.B, self.Hkv, self.Nk, self.d)

    def flops(self) -> float:
        """4*B*Hq*Nq*Nk*d, halved under the causal mask."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once (bf16) + O written once (bf16) + LSE (fp32)."""
        q = self.B * self.Hq * self.Nq * self.d * 2
        kv = 2 * self.B * self.Hkv * self.Nk * self.d * 2
        o = self.B * self.Hq * self.Nq * self.d * 2
        lse = self.B * self.Hq * self.Nq * 4
        return q + kv + o + lse

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads: the pages' benchmark shape (page 4, benchmark table:
# bs=1, heads=8, q=4096, kv=8192, BF16, head_dim 128) and four companions.
WORKLOADS = {
    "single_head_n256_d64": Workload("single_head_n256_d64", 1, 1, 1, 256, 256, 64),
    "batched_prefill_b4h16_n2048": Workload("batched_prefill_b4h16_n2048", 4, 16, 16, 2048, 2048, 128),
    "batched_prefill_b4h16_n2048_causal": Workload(
        "batched_prefill_b4h16_n2048_causal", 4, 16, 16, 2048, 2048, 128, causal=True),
    "pages_shape_h8_q4096_kv8192": Workload("pages_shape_h8_q4096_kv8192", 1, 8, 8, 4096, 8192, 128),
    "long_causal_h32_n16384": Workload("long_causal_h32_n16384", 1, 32, 32, 16384, 16384, 128, causal=True),
    "pages_shape_d256_h8_q4096_kv8192": Workload(
        "pages_shape_d256_h8_q4096_kv8192", 1, 8, 8, 4096, 8192, 256,
        note="the pages' shape at head size 256"),
    "pages_shape_d192_h8_q4096_kv8192": Workload(
        "pages_shape_d192_h8_q4096_kv8192", 1, 8, 8, 4096, 8192, 192,
        note="the pages' shape at head size 192"),
    "pages_shape_fp8_h8_q4096_kv8192": Workload(
        "pages_shape_fp8_h8_q4096_kv8192", 1, 8, 8, 4096, 8192, 128,
        note="the pages' shape with OCP E4M3 inputs and per-tensor descale factors"),
    "gqa_decode_b64_hq32_hkv8_kv8192": Workload(
        "gqa_decode_b64_hq32_hkv8_kv8192", 64, 32, 8, 1, 8192, 128, num_splits=16),
}


def _slab(seed: int, tensor: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, b, h])))
    return gen.standard_normal((n, d), dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest-even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# Per-tensor descale factors of the fp8 inputs (Q, K, V).
FP8_DESCALE = (6.75 / 448.0, 6.5 / 448.0, 6.25 / 448.0)


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode finite values as OCP E4M3 bytes (round to nearest, ties to even;
    magnitudes above 448 saturate to 448).  Returns uint8 codes, never the
    NaN codes 0x7F / 0xFF."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    # Spacing of representable values around a: 2^(e-3) for a in [2^e, 2^(e+1)),
    # e >= -6; below 2^-6 the subnormal spacing 2^-9.
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    r = np.rint(a / quantum) * quantum  # rint: ties to even (exact: quantum is a power of two)
    r = np.minimum(r, 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = r < 2.0 ** -6
    code[sub] = np.rint(r[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    with np.errstate(divide="ignore"):
        en = np.floor(np.log2(np.where(nrm, r, 1.0)))
    mant = np.rint((r / np.exp2(en) - 1.0) * 8.0).astype(np.int64)
    code[nrm] = ((en[nrm].astype(np.int64) + 7) << 3) | mant[nrm]
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw(seed: int, tensor: int, shape, heads=None, rows=None) -> np.ndarray:
    """fp32 draws for a [B, H, N, d] tensor (optionally only some heads / rows).

    ``heads``: iterable of (b, h) pairs to draw (others are not drawn; the result
    then has shape [len(heads), N, d]).  ``rows``: index array of the N axis to keep.
    """
    B, H, N, d = shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)

    def one(bh):
        s = _slab(seed, tensor, bh[0], bh[1], N, d)
        return s if rows is None else s[rows]

    if len(pairs) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            slabs = list(ex.map(one, pairs))
    else:
        slabs = [one(p) for p in pairs]
    out = np.stack(slabs, axis=0)
    if heads is None:
        out = out.reshape(B, H, out.shape[-2], d)
    return out


def draw_bf16(seed: int, tensor: int, shape, heads=None, rows=None) -> np.ndarray:
    """bf16 bit patterns (uint16) of :func:`draw`, rounded slab by slab."""
    B, H, N, d = shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)

    def one(bh):
        s = _slab(seed, tensor, bh[0], bh[1], N, d)
        return bf16_bits(s if rows is None else s[rows])

    if len(pairs) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            slabs = list(ex.map(one, pairs))
    else:
        slabs = [one(p) for p in pairs]
    out = np.stack(slabs, axis=0)
    if heads is None:
        out = out.reshape(B, H, out.shape[-2], d)
    return out


def draw_e4m3(seed: int, tensor: int, shape, heads=None, rows=None) -> np.ndarray:
    """E4M3 codes (uint8) of :func:`draw` divided by ``FP8_DESCALE[tensor]``."""
    B, H, N, d = shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    ds = FP8_DESCALE[tensor]

    def one(bh):
        s = _slab(seed, tensor, bh[0], bh[1], N, d)
        return e4m3_bits((s if rows is None else s[rows]).astype(np.float64) / ds)

    if len(pairs) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            slabs = list(ex.map(one, pairs))
    else:
        slabs = [one(p) for p in pairs]
    out = np.stack(slabs, axis=0)
    if heads is None:
        out = out.reshape(B, H, out.shape[-2], d)
    return out


def inputs_f64(w: Workload, bf16: bool = True, q_heads=None, kv_heads=None, q_rows=None):
    """(q, k, v) as float64 arrays holding exactly the values the GPU receives.

    With ``bf16`` the values are the bf16-rounded draws widened exactly; without,
    the raw fp32 draws.  ``q_heads``/``kv_heads`` restrict the (b, h) slabs drawn;
    ``q_rows`` restricts the query rows.
    """
    def get(t, shape, heads, rows=None):
        if bf16:
            return bf16_bits_to_f32(draw_bf16(w.seed, t, shape, heads, rows)).astype(np.float64)
        return draw(w.seed, t, shape, heads, rows).astype(np.float64)

    q = get(TENSOR_Q, w.q_shape, q_heads, q_rows)
    k = get(TENSOR_K, w.kv_shape, kv_heads)
    v = get(TENSOR_V, w.kv_shape, kv_heads)
    return q, k, v


def page_table(B: int, max_pages: int, seed: int, spare: int = 0):
    """A paged K/V layout: the physical page of each (sequence, logical page),
    a seeded random permutation of B * max_pages + spare pages (the spare ones
    stay unused).  Returns (num_pages, table int32 [B, max_pages])."""
    r = np.random.default_rng([seed, 0x9A6E])
    num_pages = B * max_pages + spare
    perm = r.permutation(num_pages).astype(np.int32)
    return num_pages, perm[: B * max_pages].reshape(B, max_pages)
