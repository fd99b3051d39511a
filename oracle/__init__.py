"""CPU oracle for exact attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library and its
Python binding never import, call or link anything here, and nothing here
imports them.

Parity status of each function (the pins live in tests/test_oracle.py):

* ``attention``         -- pinned (brute force, library cross-check, closed forms,
                           invariants).
* ``attention_online``  -- pinned (equals ``attention`` and the brute force for
                           several tile widths, both recurrence forms).
* ``split_bounds``, ``splitkv_partials``, ``combine`` -- pinned (combine of the
                           partials equals unsplit attention; one split is the
                           identity; empty chunks get weight zero).
* ``paged_gather``, ``paged_attention`` -- pinned (a cache built from contiguous
                           K/V under any page permutation gives back those K/V
                           and their attention; truncated lengths equal
                           attention over the first keys; brute force on a
                           tiny case).
* ``e4m3_decode``, ``e4m3_value`` -- pinned (closed-form codes of the OCP E4M3
                           format; every code against torch's float8_e4m3fn
                           conversion; monotonic over the positive codes).
* ``attention_fp8``     -- pinned through ``e4m3_decode`` and ``attention``, plus
                           the descale invariances (Q and K descales act as a
                           factor on the score scale, the V descale as a factor
                           on O).
* ``attention_backward`` -- pinned (central finite differences of <O, dO>
                           on tiny cases, torch autograd of the float64
                           definition with the same mask, the identities
                           sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, V = 1
                           giving dQ = dK = 0, D = rowsum(dO * O)).
* ``attention_backward_head`` -- the per-head step of ``attention_backward``
                           (same code path, so the pins above cover it); its
                           P and dP are also pinned directly (rows of P sum to
                           one, P equals softmax(S) from ``attention``'s LSE,
                           dP equals dO V^T).
* ``prob_weighted_abs`` -- pinned (V = 1 gives W = 1; identical keys give
                           Pmax = 1/Nk; one-hot selection gives Pmax ~ 1 and
                           W = |selected V row|; brute force on a tiny case).
"""
from .attention import (  # noqa: F401
    attention,
    attention_online,
    combine,
    paged_attention,
    paged_gather,
    split_bounds,
    splitkv_partials,
)
from .backward import attention_backward, attention_backward_head  # noqa: F401
from .fp8 import attention_fp8, e4m3_decode, e4m3_value, prob_weighted_abs  # noqa: F401
