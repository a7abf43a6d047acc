"""fa_bwd_fused_noalloc (through the C ABI) against fa_bwd_fused, the entry
point it is a variant of, and against the oracle: two calls in a row, the
second smaller than the first, so that a result of the first call left in
the shared scratch array would show up in the second."""

import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_26_amd as fa
import oracle
from workloads import cast_io, make_inputs, make_rect_inputs, to_f64

pytestmark = pytest.mark.gpu

GRAD_TOL = {"bf16": 3e-2, "fp32": 1e-4}


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _run_both(arrays, dtype, causal, window=0):
    q, k, v, do = cast_io(arrays, dtype, "cuda")
    o, lse = fa.forward(q, k, v, causal, window=window)
    delta = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    fa.fa_bwd_preprocess(o, do, delta)
    nbytes = fa.fa_bwd_fused_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], fa.FA_BF16 if dtype == "bf16" else fa.FA_F32)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda") if nbytes else None
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd_fused(q, k, v, do, lse, delta, *ref, ws, causal, window=window)
    got = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd_fused_noalloc(q, k, v, do, lse, delta, *got, causal, window=window)
    torch.cuda.synchronize()
    return [to_f64(t) for t in (q, k, v, do)], [to_f64(t) for t in ref], [to_f64(t) for t in got]


def _check(arrays, dtype, causal, window=0, label=""):
    (q, k, v, do), ref, got = _run_both(arrays, dtype, causal, window)
    oracle_grads = oracle.attention_backward(q, k, v, do, causal=causal, window=window)[:3]
    rep = {}
    for name, r, g, o in zip(("dq", "dk", "dv"), ref, got, oracle_grads):
        assert np.all(np.isfinite(g)), name
        rep[name] = np.abs(g - r).max() / np.abs(r).max()
        rep[name + "_oracle"] = np.abs(g - o).max() / np.abs(o).max()
    _say(f"[noalloc {label}] " + " ".join(f"{a}={b:.2e}" for a, b in rep.items()))
    # dK and dV come from the same kernel and arithmetic, with no atomics
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])
    for name in ("dq", "dk", "dv"):
        assert rep[name] <= GRAD_TOL[dtype], (name, rep)
        assert rep[name + "_oracle"] <= GRAD_TOL[dtype], (name, rep)


def test_noalloc_two_calls_second_smaller():
    _check(make_inputs(4, 1000, 128, seed=70), "bf16", True, label="bf16 4x1000x128 causal")
    _check(make_inputs(2, 333, 64, seed=71), "bf16", False, label="bf16 2x333x64 non-causal")


def test_noalloc_rect_window_then_smaller():
    _check(make_rect_inputs(2, 300, 1000, 128, seed=72), "bf16", True, window=100, label="bf16 rect 300x1000 window 100")
    _check(make_rect_inputs(1, 37, 100, 64, seed=73), "bf16", True, label="bf16 rect 37x100")


def test_noalloc_fp32_needs_no_scratch():
    _check(make_inputs(2, 200, 32, seed=74), "fp32", True, label="fp32 2x200x32 causal")


def test_noalloc_headline_size_fits():
    """BH 32 x N 8192 x d 128 needs exactly the whole scratch (128 MiB)."""
    assert 32 * 8192 * 128 * 4 == fa.FA_NOALLOC_SCRATCH_BYTES
    (q, k, v, do), ref, got = _run_both(make_inputs(32, 8192, 128, seed=75), "bf16", True)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])
    err = np.abs(got[0] - ref[0]).max() / np.abs(ref[0]).max()
    _say(f"[noalloc 32x8192x128] dq vs fa_bwd_fused {err:.2e}")
    assert err <= GRAD_TOL["bf16"]
