"""Whole-head oracle results for the GPU parity tests, one head at a time.

Each head runs the direct fp64 definition (``oracle.attention_forward`` and
``oracle.attention_backward``) with the BLAS library's own threads; heads are
never computed concurrently: BLAS calls issued from several host threads at
once returned wrong products on the GPU hosts (checked against single-row
oracle values), so a concurrent pool is not a trustworthy referee.
"""

from __future__ import annotations

import oracle


def head_refs(heads, causal, window=0, scale=None):
    """Yield (index, (O, L, dQ, dK, dV)) for each (q, k, v, do) fp64 head in
    `heads`, in order."""
    for i, (q, k, v, do) in enumerate(heads):
        o, lse = oracle.attention_forward(q, k, v, scale=scale, causal=causal, window=window)
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal, window=window)
        yield i, (o, lse, dq, dk, dv)
