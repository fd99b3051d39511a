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
