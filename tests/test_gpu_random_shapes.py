"""Seeded random shapes through every bf16 and float32 path against the
oracle: query and key lengths (equal or not, ragged against every tile),
head dims, causal or not, windows, every tiling, and the single-kernel
backward.  The shapes are drawn once from a fixed seed, so the cases are
the same on every run; each is small enough for the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_26_amd as fa
import oracle
from workloads import cast_io, make_rect_inputs, to_f64

pytestmark = pytest.mark.gpu

TOL = {"fp32": dict(o=1e-5, lse=1e-5, grad=1e-4), "bf16": dict(o=1e-2, lse=1e-3, grad=3e-2)}
BF16_TILES = {128: dict(fwd=[(256, 64), (128, 64)], dkdv=[(128, 128), (64, 128)], dq=[(256, 32), (128, 32), (128, 64)]),
              64: dict(fwd=[(128, 64), (256, 64)], dkdv=[(128, 128), (64, 128)], dq=[(128, 64), (128, 32), (256, 64)])}
F32_TILES = [(16, 12), (32, 64), (64, 32), (128, 64), (64, 64), (16, 128)]


def _cases(count=120, seed=123):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        dtype = "bf16" if c % 3 else "fp32"
        d = int(rng.choice([64, 128])) if dtype == "bf16" else int(rng.choice([16, 32, 64, 128]))
        nk = int(rng.integers(1, 700))
        causal = bool(rng.integers(0, 2))
        nq = int(rng.integers(1, nk + 1)) if causal else int(rng.integers(1, 700))
        if rng.random() < 0.3:
            nq = nk
        window = int(rng.integers(1, nk + 40)) if causal and rng.random() < 0.4 else 0
        fused = bool(rng.random() < 0.25)
        bh = int(rng.integers(1, 4))
        if dtype == "bf16":
            t = BF16_TILES[d]
            tiles = tuple(t[k][int(rng.integers(0, len(t[k])))] for k in ("fwd", "dkdv", "dq"))
            if fused:
                tiles = (tiles[0], (64, 128), tiles[2])   # the fused backward's bf16 tiling
        else:
            tiles = tuple(F32_TILES[int(rng.integers(0, len(F32_TILES)))] for _ in range(3))
        out.append((c, dtype, bh, nq, nk, d, causal, window, fused, tiles))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    c, dtype, bh, nq, nk, d, causal, window, fused, tiles = case
    label = (f"case {c}: {dtype} bh={bh} nq={nq} nk={nk} d={d} causal={causal} window={window} "
             f"fused={fused} tiles={tiles}")
    print(label, file=sys.stderr, flush=True)
    arrays = make_rect_inputs(bh, nq, nk, d, seed=1000 + c)
    q, k, v, do = cast_io(arrays, dtype, "cuda")
    o, lse = fa.forward(q, k, v, causal, None, *tiles[0], window=window)
    if fused:
        dq, dk, dv, _ = fa.backward_fused(q, k, v, o, do, lse, causal, None, tiles[1], window=window)
    else:
        dq, dk, dv, _ = fa.backward(q, k, v, o, do, lse, causal, None, tiles[1], tiles[2], window=window)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o_ref, l_ref = oracle.attention_forward(q64, k64, v64, causal=causal, window=window)
    g_ref = oracle.attention_backward(q64, k64, v64, do64, causal=causal, window=window)
    tol = TOL[dtype]
    assert np.abs(to_f64(o) - o_ref).max() <= tol["o"], label
    assert np.abs(to_f64(lse) - l_ref).max() <= tol["lse"], label
    for name, got, ref in (("dq", dq, g_ref[0]), ("dk", dk, g_ref[1]), ("dv", dv, g_ref[2])):
        scale = max(np.abs(ref).max(), 1.0 if np.abs(ref).max() == 0 else 0.0)
        assert np.abs(to_f64(got) - ref).max() <= tol["grad"] * scale, (name, label)
