"""torch autograd drop-in for exact tiled attention.

``flash_attention(q, k, v, causal=False, scale=None, window=0)`` computes
``softmax(scale * q k^T) v`` (keys after the query masked when ``causal``)
with the library's kernels and differentiates through them.  Following
"Assignment2: FlashAttention & Distributed Data Parallel notes" (CS336)
section 1.2, the forward saves only Q, K, V, O and the logsumexp L (one
float per row, no N x N matrix); section 1.4's backward then runs
``fa_bwd_preprocess`` (D = rowsum(O * dO)), ``fa_bwd_dkdv`` and ``fa_bwd_dq``
on the current stream.

Inputs are device tensors of one dtype (float32 or bfloat16): q of shape
``[..., nq, d]`` and k, v of shape ``[..., nk, d]`` with the same leading
dimensions, which are flattened into the kernels' head axis.  With nq != nk
the causal mask is aligned to the end of the keys (query i sees keys
0 .. i + nk - nq, e.g. new tokens against a key/value cache).  ``window`` > 0
(causal only) further limits each query to its ``window`` most recent keys,
as in "CS324 lecture 8, 03_online_softmax_and_flash.py"'s window_attention_torch.  Gradients
come back in the input dtype.  There is no fallback: the kernels run or the
call raises.
"""

from __future__ import annotations

import torch

from . import _lib


def _flat(t: torch.Tensor) -> torch.Tensor:
    return t.reshape(-1, t.shape[-2], t.shape[-1]).contiguous()


class FlashAttention(torch.autograd.Function):
    """Autograd function over ``fa_fwd`` and the three backward calls."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float | None, window: int = 0):
        if q.dim() < 3 or k.dim() != q.dim():
            raise ValueError(f"expected [..., n, d] tensors, got shapes {tuple(q.shape)}, {tuple(k.shape)}")
        if k.shape != v.shape or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != q.shape[-1]:
            raise ValueError(f"k and v must be [..., nk, d] with q's leading dims and d, got "
                             f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
        q3, k3, v3 = _flat(q), _flat(k), _flat(v)
        o, lse = _lib.forward(q3, k3, v3, causal, scale, window=int(window))
        ctx.save_for_backward(q3, k3, v3, o, lse)
        ctx.causal = bool(causal)
        ctx.window = int(window)
        ctx.scale = scale
        ctx.shapes = (q.shape, k.shape)
        return o.view(q.shape)

    @staticmethod
    def backward(ctx, do):
        q3, k3, v3, o, lse = ctx.saved_tensors
        do3 = do.to(o.dtype).reshape(o.shape).contiguous()
        dq, dk, dv, _ = _lib.backward(q3, k3, v3, o, do3, lse, ctx.causal, ctx.scale,
                                      window=ctx.window)
        qshape, kshape = ctx.shapes
        return dq.view(qshape), dk.view(kshape), dv.view(kshape), None, None, None


def flash_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    scale: float | None = None, window: int = 0) -> torch.Tensor:
    """Exact attention with the library's kernels; differentiable in q, k, v.

    ``scale`` defaults to 1/sqrt(d) and must be finite and positive;
    ``window`` is 0 (none) or a positive key count with ``causal``."""
    return FlashAttention.apply(q, k, v, causal, scale, window)
