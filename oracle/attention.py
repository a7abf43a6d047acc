"""Direct fp64 definition of exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method is exact: tiling and the online softmax change only the order of
the arithmetic, not the function ([CS324-L8] header and demo3_forward
observations).  So the oracle is the textbook computation written out with
the full score matrix of each head, in fp64:

1. ``S = scale * Q K^T``                       ([CS336-A2] 1.1; 1.4 Eq 13)
2. causal: ``S_ij = -inf`` for key ``j > i``    ([CS324-L8] demo4_backward,
   lower-triangular ``tril`` mask; query ``i`` sees keys ``0..i``).  With
   ``N_q`` queries against ``N_k >= N_q`` keys the queries are the last
   ``N_q`` positions: key ``j`` is masked iff ``j > i + (N_k - N_q)`` (the
   decode remark of [CS349E-L11] demo4_causal: one new query sees every
   cached key); ``N_q = N_k`` is the square case.  A sliding window of
   ``w`` keys ([CS324-L8] window_attention_torch: a row sees itself and the
   ``w - 1`` keys before it) additionally masks ``j <= i + (N_k - N_q) - w``.
3. ``m_i = max_j S_ij``, ``L_i = m_i + ln sum_j exp(S_ij - m_i)``
   (the logsumexp saved by the forward, [CS336-A2] 1.2)
4. ``P = exp(S - L)``                          ([CS336-A2] 1.4 Eq 14)
5. ``O = P V``
6. ``dV = P^T dO``                             (Eq 15)
7. ``dP = dO V^T``                             (Eq 16)
8. ``D_i = sum_j P_ij dP_ij``                  (the definition of D in Eq 17)
9. ``dS = P * (dP - D)``                       (Eq 17)
10. ``dQ = scale * dS K``                      (Eq 18)
11. ``dK = scale * dS^T Q``                    (Eq 19)

The pages only use ``scale = 1/sqrt(d)``; the scale is an explicit argument
here and multiplies both dQ and dK.  Rows are processed in chunks of whole
rows (each chunk still sees the full row of S), which only regroups the sums
that build dK and dV.  Inputs may be any float dtype; they are upcast to fp64
first, so the oracle sees exactly the values the GPU sees.
"""

from __future__ import annotations

import math

import numpy as np

DEFAULT_CHUNK = 1024


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _check_window(causal: bool, window: int) -> int:
    window = int(window)
    if window < 0 or (window and not causal):
        raise ValueError(f"a sliding window needs causal masking and window >= 1 (got {window})")
    return window


def _causal_offset(nq: int, nk: int, causal: bool) -> int:
    """Shift of the causal diagonal: query i sees keys 0 .. i + (nk - nq)."""
    if not causal:
        return 0
    if nq > nk:
        raise ValueError(f"causal attention needs at least as many keys as queries (nq={nq}, nk={nk})")
    return nk - nq


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float, causal: bool,
            row_idx: np.ndarray, col_idx: np.ndarray | None = None, offset: int = 0,
            window: int = 0) -> np.ndarray:
    """Steps 1-2: scaled scores of the given query rows against keys ``col_idx``
    (all keys when None), with the causal mask applied by global index
    (key j visible to query i iff j <= i + offset, and j > i + offset - window
    when window > 0)."""
    if col_idx is None:
        col_idx = np.arange(k.shape[0])
    s = scale * (q_rows @ k.T)
    if causal:
        hidden = col_idx[None, :] > row_idx[:, None] + offset
        if window:
            hidden |= col_idx[None, :] <= row_idx[:, None] + offset - window
        s = np.where(hidden, -np.inf, s)
    return s


def _logsumexp_rows(s: np.ndarray) -> np.ndarray:
    """Step 3: L_i = m_i + ln sum_j exp(S_ij - m_i), with the row max m_i
    subtracted first so that no exponent overflows ([CS324-L8]
    demo1_overflow: the max-subtracted, "safe" softmax)."""
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def _forward_head(q, k, v, scale, causal, chunk, window=0):
    n = q.shape[0]
    off = _causal_offset(n, k.shape[0], causal)
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = _scores(q[rows], k, scale, causal, rows, offset=off, window=window)
        lse[rows] = _logsumexp_rows(s)
        p = np.exp(s - lse[rows][:, None])            # step 4
        o[rows] = p @ v                                 # step 5
    return o, lse


def _backward_head(q, k, v, do, scale, causal, chunk, window=0):
    n = q.shape[0]
    off = _causal_offset(n, k.shape[0], causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = _scores(q[rows], k, scale, causal, rows, offset=off, window=window)
        lse = _logsumexp_rows(s)
        p = np.exp(s - lse[:, None])                    # step 4
        dv += p.T @ do[rows]                            # step 6
        dp = do[rows] @ v.T                             # step 7
        delta[rows] = (p * dp).sum(axis=1)              # step 8
        ds = p * (dp - delta[rows][:, None])            # step 9
        dq[rows] = scale * (ds @ k)                     # step 10
        dk += scale * (ds.T @ q[rows])                  # step 11
    return dq, dk, dv, delta


def _batched(fn, arrays, *args):
    """Apply a per-head function to [N, d] or [BH, N, d] inputs."""
    arrays = [_f64(a) for a in arrays]
    if arrays[0].ndim == 2:
        return fn(*arrays, *args)
    outs = [fn(*[a[h] for a in arrays], *args) for h in range(arrays[0].shape[0])]
    return tuple(np.stack(parts) for parts in zip(*outs))


def attention_forward(q, k, v, scale=None, causal=False, chunk=DEFAULT_CHUNK, window=0):
    """Return ``(O, L)`` for q of shape [N_q, d] or [BH, N_q, d] and k, v of
    shape [N_k, d] or [BH, N_k, d] (fp64).  ``window`` > 0 (causal only)
    limits each query to its ``window`` most recent keys."""
    scale = _default_scale(np.shape(q)[-1], scale)
    window = _check_window(causal, window)
    return _batched(_forward_head, (q, k, v), scale, bool(causal), int(chunk), window)


def attention_backward(q, k, v, do, scale=None, causal=False, chunk=DEFAULT_CHUNK, window=0):
    """Return ``(dQ, dK, dV, D)`` for the loss whose gradient w.r.t. O is dO.

    D is computed by its definition ``sum_j P_ij dP_ij``; the forward output
    is not needed.
    """
    scale = _default_scale(np.shape(q)[-1], scale)
    window = _check_window(causal, window)
    return _batched(_backward_head, (q, k, v, do), scale, bool(causal), int(chunk), window)


def delta_from_output(o, do):
    """``D_i = sum_k dO_ik O_ik``: the identity that lets D be computed from
    one row of O and dO before the backward starts ([CS336-A2] 1.4 Eq 17;
    [CS349E-L11] demo1_gradcheck observations)."""
    return (_f64(o) * _f64(do)).sum(axis=-1)


# --------------------------------------------------------------------------
# Sampled outputs for large inputs: each value below is computed one by one
# from the same definition, without forming any other row's outputs.
# --------------------------------------------------------------------------

def forward_rows(q, k, v, rows, scale=None, causal=False, window=0):
    """O[rows] and L[rows] of one head (q, k, v: [N, d]).  A row of the
    forward depends only on that row's scores."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    scale = _default_scale(q.shape[1], scale)
    rows = np.asarray(rows, dtype=np.int64)
    s = _scores(q[rows], k, scale, causal, rows, offset=_causal_offset(q.shape[0], k.shape[0], causal),
                window=_check_window(causal, window))
    lse = _logsumexp_rows(s)
    return np.exp(s - lse[:, None]) @ v, lse


def dq_rows(q, k, v, do, rows, scale=None, causal=False, window=0):
    """dQ[rows] and D[rows] of one head.  Row i of dQ needs only row i of
    S, P, dP and dS (steps 1-4, 7-10)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    scale = _default_scale(q.shape[1], scale)
    rows = np.asarray(rows, dtype=np.int64)
    s = _scores(q[rows], k, scale, causal, rows, offset=_causal_offset(q.shape[0], k.shape[0], causal),
                window=_check_window(causal, window))
    p = np.exp(s - _logsumexp_rows(s)[:, None])
    dp = do[rows] @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    return scale * (ds @ k), delta


def head_row_stats(q, k, v, do, scale=None, causal=False, chunk=DEFAULT_CHUNK, window=0):
    """L and D for every row of one head (full rows, in chunks)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    scale = _default_scale(q.shape[1], scale)
    n = q.shape[0]
    off = _causal_offset(n, k.shape[0], causal)
    window = _check_window(causal, window)
    lse = np.empty(n)
    delta = np.empty(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = _scores(q[rows], k, scale, causal, rows, offset=off, window=window)
        lse[rows] = _logsumexp_rows(s)
        p = np.exp(s - lse[rows][:, None])
        delta[rows] = (p * (do[rows] @ v.T)).sum(axis=1)
    return lse, delta


def dkdv_cols(q, k, v, do, cols, scale=None, causal=False, stats=None,
              chunk=DEFAULT_CHUNK, window=0):
    """dK[cols] and dV[cols] of one head.  Column j of dK/dV sums over every
    query row, so it needs L_i and D_i of all rows (``stats`` = the pair
    returned by :func:`head_row_stats`; computed here when None) and then only
    column j of P, dP and dS (steps 4, 6-9, 11)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    scale = _default_scale(q.shape[1], scale)
    cols = np.asarray(cols, dtype=np.int64)
    if stats is None:
        stats = head_row_stats(q, k, v, do, scale, causal, chunk, window)
    lse, delta = stats
    n = q.shape[0]
    off = _causal_offset(n, k.shape[0], causal)
    window = _check_window(causal, window)
    dk = np.zeros((len(cols), k.shape[1]))
    dv = np.zeros((len(cols), v.shape[1]))
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = _scores(q[rows], k[cols], scale, causal, rows, cols, offset=off, window=window)
        p = np.exp(s - lse[rows][:, None])
        dv += p.T @ do[rows]
        dp = do[rows] @ v[cols].T
        ds = p * (dp - delta[rows][:, None])
        dk += scale * (ds.T @ q[rows])
    return dk, dv
