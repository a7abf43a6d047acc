"""fp64 CPU model of the tiled algorithm, used to check the pages' claims.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It is compared with
``oracle.attention`` (the direct definition), never with the GPU.

* :func:`online_softmax` -- the running max ``m`` and running denominator
  ``l`` read block by block ([CS324-L8] demo2_online; [CS336-A2] 1.2).
* :func:`tiled_forward` -- the FA-2 forward of [CS336-A2] 1.2: per query tile
  an unnormalised accumulator rescaled by ``exp(m - m_new)``, a single divide
  by ``l`` at the end, and ``L = m + log l`` saved.  Causal mode skips key
  tiles that start after the tile's last query row ([CS336-A2] 1.3) and masks
  inside tiles that cross the diagonal ([CS324-L8] flash_attention_torch).
* :func:`tiled_backward` -- Eq 13-19 of [CS336-A2] 1.4 in two passes: one
  with the outer loop over key/value tiles (accumulates dK, dV) and one with
  the outer loop over query tiles (accumulates dQ), each recomputing
  ``P = exp(S - L)``; ``D = rowsum(O * dO)`` is formed first.
* :func:`causal_tiles_computed` -- how many (query tile, key tile) pairs the
  causal skip rule leaves ([CS349E-L11] demo4_causal).

Ragged last tiles are smaller, as the flash_attention_torch docstring of
[CS324-L8] describes.
"""

from __future__ import annotations

import math

import numpy as np


def online_softmax(x, block: int, trace: bool = False):
    """Softmax of a vector read ``block`` entries at a time, keeping only the
    running max ``m`` and the running denominator ``l`` (relative to ``m``).

    On each block: ``m_new = max(m, max(block))`` and
    ``l <- l * exp(m - m_new) + sum(exp(block - m_new))``.  Before the first
    block ``m = -inf`` and ``l = 0``, so the first rescale factor is 0.
    Returns the softmax, and with ``trace`` also a list of
    ``(entries read so far, m, l)`` after each block.
    """
    x = np.asarray(x, dtype=np.float64)
    m, l = -np.inf, 0.0
    steps = []
    for start in range(0, x.size, block):
        blk = x[start:start + block]
        m_new = max(m, float(blk.max()))
        corr = 0.0 if m == -np.inf else math.exp(m - m_new)
        l = l * corr + float(np.exp(blk - m_new).sum())
        m = m_new
        steps.append((start + blk.size, m, l))
    out = np.exp(x - m) / l
    return (out, steps) if trace else out


def _tile_visible(i0: int, ni: int, j0: int) -> bool:
    """A key tile starting at ``j0`` holds at least one key visible to the
    query tile ``[i0, i0 + ni)`` iff ``j0 <= i0 + ni - 1`` (its first key is
    not after the tile's last query)."""
    return j0 <= i0 + ni - 1


def _mask_tile(s, i0, ni, j0, nj):
    rows = np.arange(i0, i0 + ni)[:, None]
    cols = np.arange(j0, j0 + nj)[None, :]
    return np.where(cols > rows, -np.inf, s)


def tiled_forward(q, k, v, br: int, bc: int, scale=None, causal=False):
    """FA-2 forward over Br x Bc tiles of one head.

    Returns ``(O, L, tiles)`` where ``tiles`` counts the (query tile, key
    tile) pairs actually computed.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    tiles = 0
    for i0 in range(0, n, br):
        qi = q[i0:i0 + br]
        ni = qi.shape[0]
        acc = np.zeros((ni, v.shape[1]))
        l = np.zeros(ni)
        m = np.full(ni, -np.inf)
        for j0 in range(0, n, bc):
            if causal and not _tile_visible(i0, ni, j0):
                break                       # every later key tile is masked too
            kj, vj = k[j0:j0 + bc], v[j0:j0 + bc]
            nj = kj.shape[0]
            s = scale * (qi @ kj.T)
            if causal and j0 + nj - 1 > i0:  # tile crosses the diagonal
                s = _mask_tile(s, i0, ni, j0, nj)
            m_new = np.maximum(m, s.max(axis=1))
            # rows that have seen no visible key yet keep a zero contribution
            safe = np.where(m_new == -np.inf, 0.0, m_new)
            p = np.exp(s - safe[:, None])
            corr = np.where(m == -np.inf, 0.0, np.exp(m - safe))
            l = corr * l + p.sum(axis=1)
            acc = corr[:, None] * acc + p @ vj
            m = m_new
            tiles += 1
        o[i0:i0 + ni] = acc / l[:, None]
        lse[i0:i0 + ni] = m + np.log(l)
    return o, lse, tiles


def tiled_backward(q, k, v, o, do, lse, br: int, bc: int, scale=None,
                   causal=False):
    """Two-pass tiled backward of one head from (Q, K, V, O, dO, L).

    Returns ``(dQ, dK, dV, D, tiles_kv_pass, tiles_q_pass)``.
    """
    q, k, v, o, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, dtype=np.float64)
    n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    delta = (o * do).sum(axis=1)          # D before the backward starts

    def probs(i0, ni, j0, nj):
        s = scale * (q[i0:i0 + ni] @ k[j0:j0 + nj].T)             # Eq 13
        if causal and j0 + nj - 1 > i0:
            s = _mask_tile(s, i0, ni, j0, nj)
        return np.exp(s - lse[i0:i0 + ni][:, None])              # Eq 14

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    tiles_kv = tiles_q = 0
    # pass 1: outer loop over key/value tiles accumulates dK_j and dV_j
    for j0 in range(0, n, bc):
        nj = min(bc, n - j0)
        dkj = np.zeros((nj, d))
        dvj = np.zeros((nj, v.shape[1]))
        for i0 in range(0, n, br):
            ni = min(br, n - i0)
            if causal and not _tile_visible(i0, ni, j0):
                continue
            p = probs(i0, ni, j0, nj)
            dvj += p.T @ do[i0:i0 + ni]                              # Eq 15
            dp = do[i0:i0 + ni] @ v[j0:j0 + nj].T                    # Eq 16
            ds = p * (dp - delta[i0:i0 + ni][:, None])               # Eq 17
            dkj += scale * (ds.T @ q[i0:i0 + ni])                    # Eq 19
            tiles_kv += 1
        dk[j0:j0 + nj] = dkj
        dv[j0:j0 + nj] = dvj
    # pass 2: outer loop over query tiles accumulates dQ_i
    for i0 in range(0, n, br):
        ni = min(br, n - i0)
        dqi = np.zeros((ni, d))
        for j0 in range(0, n, bc):
            if causal and not _tile_visible(i0, ni, j0):
                break
            nj = min(bc, n - j0)
            p = probs(i0, ni, j0, nj)
            dp = do[i0:i0 + ni] @ v[j0:j0 + nj].T
            ds = p * (dp - delta[i0:i0 + ni][:, None])
            dqi += scale * (ds @ k[j0:j0 + nj])                      # Eq 18
            tiles_q += 1
        dq[i0:i0 + ni] = dqi
    return dq, dk, dv, delta, tiles_kv, tiles_q


def causal_tiles_computed(n: int, br: int, bc: int) -> int:
    """Number of (query tile, key tile) pairs the causal skip rule keeps."""
    count = 0
    for i0 in range(0, n, br):
        ni = min(br, n - i0)
        for j0 in range(0, n, bc):
            if _tile_visible(i0, ni, j0):
                count += 1
    return count
