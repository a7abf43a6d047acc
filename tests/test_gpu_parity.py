"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.

Tolerances (float32 I/O): |O - O_ref| <= 1e-5 and |L - L_ref| <= 1e-5
absolute; max |dX - dX_ref| <= 1e-4 * max |dX_ref| for X in Q, K, V.
(bf16 I/O, fp32 accumulation): |O - O_ref| <= 1e-2, |L - L_ref| <= 1e-3;
gradients <= 3e-2 * max |dX_ref|.  The oracle reads the exact values of the
cast I/O tensors (upcast to fp64), so input rounding is not charged to the
kernels.
"""

import math
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_26_amd as fa
import oracle
from workloads import WORKLOADS, cast_io, make_inputs, make_rect_inputs, to_f64

pytestmark = pytest.mark.gpu

TOL = {
    "fp32": dict(o=1e-5, lse=1e-5, grad=1e-4, delta=1e-5),
    "bf16": dict(o=1e-2, lse=1e-3, grad=3e-2, delta=1e-2),
}


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def run_gpu(arrays, dtype, causal, fwd_tiles=(0, 0), dkdv_tiles=(0, 0), dq_tiles=(0, 0), scale=None,
            window=0):
    q, k, v, do = cast_io(arrays, dtype, "cuda")
    o, lse = fa.forward(q, k, v, causal, scale, *fwd_tiles, window=window)
    dq, dk, dv, delta = fa.backward(q, k, v, o, do, lse, causal, scale, dkdv_tiles, dq_tiles,
                                    window=window)
    torch.cuda.synchronize()
    out = {name: to_f64(t) for name, t in
           dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta).items()}
    return out


def _rel(err, ref):
    """Gradient error relative to max |ref|.  Where the exact gradient is 0
    (a single token: dQ = dK = 0) the error is taken relative to 1."""
    return err / max(np.abs(ref).max(), 1.0 if np.abs(ref).max() == 0 else 0.0)


def compare_full(g, dtype, causal, scale=None, label="", magnitude=1.0, window=0):
    """Whole-tensor comparison with the oracle; returns the error report.

    `magnitude` widens the O and L bounds for inputs whose scores are far
    larger than the N(0, 1) workloads': an fp32 logsumexp of size |L| cannot
    be closer than about |L| * 2^-24, so the bounds there are taken relative
    to the score scale.
    """
    tol = dict(TOL[dtype])
    tol["o"] *= magnitude
    tol["lse"] *= magnitude
    o_ref, l_ref = oracle.attention_forward(g["q"], g["k"], g["v"], scale=scale, causal=causal,
                                            window=window)
    dq_ref, dk_ref, dv_ref, _ = oracle.attention_backward(g["q"], g["k"], g["v"], g["do"], scale=scale,
                                                          causal=causal, window=window)
    # D from the GPU's own stored O (the identity the backward uses)
    d_ref = oracle.delta_from_output(g["o"], g["do"])
    rep = {
        "o": np.abs(g["o"] - o_ref).max(),
        "lse": np.abs(g["lse"] - l_ref).max(),
        "delta": np.abs(g["delta"] - d_ref).max() / max(1.0, np.abs(d_ref).max()),
        "dq": _rel(np.abs(g["dq"] - dq_ref).max(), dq_ref),
        "dk": _rel(np.abs(g["dk"] - dk_ref).max(), dk_ref),
        "dv": _rel(np.abs(g["dv"] - dv_ref).max(), dv_ref),
    }
    _say(f"[{label}] " + " ".join(f"{k}={v:.2e}" for k, v in rep.items()))
    assert rep["o"] <= tol["o"], rep
    assert rep["lse"] <= tol["lse"], rep
    assert rep["delta"] <= tol["delta"], rep
    for name in ("dq", "dk", "dv"):
        assert rep[name] <= tol["grad"], (name, rep)
    for name in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert np.all(np.isfinite(g[name])), name
    return rep


# --------------------------------------------------------------------------- small configs
@pytest.mark.parametrize("causal", [False, True])
def test_gradcheck_workload_16x12(causal):
    """Single head, N = 48, d = 16, fp32, tiles 16 x 12, seed 0."""
    w = WORKLOADS["gradcheck_48"]
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    g = run_gpu(arrays, "fp32", causal, (16, 12), (16, 12), (16, 12))
    compare_full(g, "fp32", causal, label=f"48x16 16x12 causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_tile_sweep(causal):
    """BH = 4, N = 256, d = 32, fp32: every tiling matches the oracle, and the
    tilings agree with each other."""
    w = WORKLOADS["tile_sweep_256"]
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    results = []
    for bm, bn in w.tiles:
        g = run_gpu(arrays, "fp32", causal, (bm, bn), (bm, bn), (bm, bn))
        compare_full(g, "fp32", causal, label=f"sweep ({bm},{bn}) causal={causal}")
        results.append(g)
    for g in results[1:]:
        for name in ("o", "lse", "dq", "dk", "dv"):
            scale = max(1.0, np.abs(results[0][name]).max())
            assert np.abs(g[name] - results[0][name]).max() <= 1e-5 * scale, name


# every bf16 d = 64 tiling: forward (128, 64) and (256, 64), dK/dV (128, 128)
# and (64, 128), dQ (128, 64) and (128, 32)
@pytest.mark.parametrize("fwd_tiles,dkdv_tiles,dq_tiles", [((128, 64), (128, 128), (128, 64)),
                                                           ((256, 64), (64, 128), (128, 32))])
def test_bf16_2048_d64_causal(fwd_tiles, dkdv_tiles, dq_tiles):
    """batch 4 x heads 8, N = 2048, d = 64, bf16, causal."""
    w = WORKLOADS["bf16_2048_d64"]
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    g = run_gpu(arrays, "bf16", True, fwd_tiles, dkdv_tiles, dq_tiles)
    compare_full(g, "bf16", True, label=f"bf16 32x2048x64 fwd{fwd_tiles} dkdv{dkdv_tiles} dq{dq_tiles}")


@pytest.mark.parametrize("dq_tiles", [(0, 0), (128, 64), (128, 32), (256, 64)])
def test_bf16_2048_d64_noncausal(dq_tiles):
    arrays = make_inputs(8, 2048, 64, seed=1)
    g = run_gpu(arrays, "bf16", False, (0, 0), (0, 0), dq_tiles)
    compare_full(g, "bf16", False, label=f"bf16 8x2048x64 non-causal dq{dq_tiles}")


# every bf16 d = 128 tiling: forward (128, 64) and (256, 64), dK/dV (64, 128)
# and (128, 128), dQ (256, 32), (128, 32) and (128, 64)
BF16_D128_TILINGS = [((128, 64), (64, 128), (128, 32)), ((256, 64), (128, 128), (128, 64)),
                     ((256, 64), (128, 128), (256, 32))]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", BF16_D128_TILINGS)
def test_bf16_d128_small(causal, tiles):
    arrays = make_inputs(4, 1024, 128, seed=2)
    g = run_gpu(arrays, "bf16", causal, *tiles)
    compare_full(g, "bf16", causal, label=f"bf16 4x1024x128 tiles={tiles} causal={causal}")


# --------------------------------------------------------------------------- ragged / edge
@pytest.mark.parametrize("n", [1, 5, 50, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_fp32(n, causal):
    arrays = make_inputs(2, n, 16, seed=3)
    for tiles in ((16, 12), (32, 64), (64, 32)):
        g = run_gpu(arrays, "fp32", causal, tiles, tiles, tiles)
        compare_full(g, "fp32", causal, label=f"fp32 n={n} tiles={tiles} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 17, 100, 333, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bf16(d, n, causal):
    arrays = make_inputs(3, n, d, seed=4)
    g = run_gpu(arrays, "bf16", causal)
    compare_full(g, "bf16", causal, label=f"bf16 n={n} d={d} causal={causal}")


@pytest.mark.parametrize("dtype,d", [("fp32", 32), ("bf16", 128)])
def test_large_scores_stay_finite(dtype, d):
    """Scores of order 1e2 (Q scaled by 50): the online softmax never
    overflows and still matches the oracle.  The O and L bounds scale with the
    largest |score| / 10 (L ~ 200 here; fp32 resolves it to ~1e-5)."""
    q, k, v, do = make_inputs(2, 300, d, seed=5)
    q = q * 50
    g = run_gpu((q, k, v, do), dtype, True)
    smax = max(np.abs(g["q"][h] @ g["k"][h].T).max() / np.sqrt(d) for h in range(2))
    compare_full(g, dtype, True, label=f"{dtype} large scores (max |S| {smax:.0f})",
                 magnitude=max(1.0, smax / 10))


def test_explicit_scale_fp32():
    arrays = make_inputs(2, 130, 32, seed=6)
    g = run_gpu(arrays, "fp32", True, (32, 16), (32, 16), (32, 16), scale=0.3)
    compare_full(g, "fp32", True, scale=0.3, label="fp32 scale=0.3")


def test_explicit_scale_bf16():
    arrays = make_inputs(2, 300, 64, seed=6)
    g = run_gpu(arrays, "bf16", False, scale=0.05)
    compare_full(g, "bf16", False, scale=0.05, label="bf16 scale=0.05")


def test_constant_v_gives_constant_output():
    """Rows of P sum to one, so V = 1 gives O = 1 and dV = column sums of P^T dO."""
    q, k, _, do = make_inputs(2, 512, 128, seed=7)
    g = run_gpu((q, k, np.ones_like(q), do), "bf16", True)
    assert np.abs(g["o"] - 1.0).max() <= 1e-2


def test_determinism_bitwise():
    """No atomics anywhere: two runs on the same inputs are bitwise identical
    (a race on LDS or a missing barrier would show up here)."""
    arrays = make_inputs(4, 2048, 128, seed=8)
    for causal in (True, False):
        a = run_gpu(arrays, "bf16", causal)
        b = run_gpu(arrays, "bf16", causal)
        for name in ("o", "lse", "dq", "dk", "dv", "delta"):
            assert np.array_equal(a[name], b[name]), name


# --------------------------------------------------------------------------- full-size, sampled
def sampled_check(w, causal, heads, rows, cols, window=0):
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    g = run_gpu(arrays, w.dtype, causal, window=window)
    tol = TOL[w.dtype]
    for h in heads:
        q, k, v, do = (g[x][h] for x in ("q", "k", "v", "do"))
        o_ref, l_ref = oracle.forward_rows(q, k, v, rows, causal=causal, window=window)
        dq_ref, d_ref = oracle.dq_rows(q, k, v, do, rows, causal=causal, window=window)
        stats = oracle.head_row_stats(q, k, v, do, causal=causal, window=window)
        dk_ref, dv_ref = oracle.dkdv_cols(q, k, v, do, cols, causal=causal, stats=stats, window=window)
        # gradient scale from the whole head's GPU gradients (the reference max
        # over the sampled entries would understate it)
        rep = {
            "o": np.abs(g["o"][h][rows] - o_ref).max(),
            "lse": np.abs(g["lse"][h][rows] - l_ref).max(),
            "dq": np.abs(g["dq"][h][rows] - dq_ref).max() / np.abs(g["dq"][h]).max(),
            "dk": np.abs(g["dk"][h][cols] - dk_ref).max() / np.abs(g["dk"][h]).max(),
            "dv": np.abs(g["dv"][h][cols] - dv_ref).max() / np.abs(g["dv"][h]).max(),
        }
        _say(f"[{w.name} causal={causal} window={window} head={h}] " +
             " ".join(f"{a}={b:.2e}" for a, b in rep.items()))
        assert rep["o"] <= tol["o"] and rep["lse"] <= tol["lse"], rep
        for name in ("dq", "dk", "dv"):
            assert rep[name] <= tol["grad"], (name, rep)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.all(np.isfinite(g[name])), name


@pytest.mark.parametrize("causal", [True, False])
def test_headline_sampled(causal):
    """BH = 32, N = 8192, d = 128, bf16 at the default tilings bench.py times."""
    w = WORKLOADS["headline_8192_d128"]
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 8191], rng.integers(0, w.n, 24)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 4096, 8190, 8191], rng.integers(0, w.n, 9)]))
    sampled_check(w, causal, heads=[0, 31], rows=rows, cols=cols)


def test_long_context_sampled_and_memory():
    """BH = 8, N = 32768, d = 128, bf16, causal; no N x N buffer is ever
    allocated (peak device memory stays at the I/O tensors)."""
    w = WORKLOADS["long_32768_d128"]
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    rng = np.random.default_rng(98)
    rows = np.unique(np.concatenate([[0, 1, 16383, 32767], rng.integers(0, w.n, 12)]))
    cols = np.unique(np.concatenate([[0, 32767], rng.integers(0, w.n, 6)]))
    sampled_check(w, True, heads=[5], rows=rows, cols=cols)
    peak = torch.cuda.max_memory_allocated() - base
    io_bytes = 9 * w.bh * w.n * w.d * 2 + 2 * w.bh * w.n * 4      # q k v do o dq dk dv + L, D
    nxn_bytes = w.bh * w.n * w.n * 2
    _say(f"peak {peak / 2**20:.1f} MiB, I/O {io_bytes / 2**20:.1f} MiB, one bf16 P would be {nxn_bytes / 2**30:.1f} GiB")
    assert peak <= io_bytes * 1.05 + (8 << 20)


# --------------------------------------------------------------------------- nq != nk
# nq queries against nk keys through the *_rect calls (the binding picks them
# when k is longer or shorter than q); causal masks are aligned to the end of
# the keys.  Sizes span several tiles with ragged ends on both axes.
# (causal with more queries than keys is rejected: test_rect_rejects_causal_with_more_queries)
def _rect_cases(shapes):
    return [(nq, nk, causal) for nq, nk in shapes for causal in (False, True) if not (causal and nq > nk)]


@pytest.mark.parametrize("nq,nk,causal", _rect_cases([(37, 100), (1, 64), (64, 200), (200, 64)]))
def test_rect_fp32(nq, nk, causal):
    arrays = make_rect_inputs(2, nq, nk, 32, seed=30)
    for tiles in ((16, 12), (64, 64)):
        g = run_gpu(arrays, "fp32", causal, tiles, tiles, tiles)
        compare_full(g, "fp32", causal, label=f"fp32 rect {nq}x{nk} tiles={tiles} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal", _rect_cases([(300, 1000), (1, 513), (256, 4096), (500, 200)]))
def test_rect_bf16(d, nq, nk, causal):
    arrays = make_rect_inputs(2, nq, nk, d, seed=31)
    g = run_gpu(arrays, "bf16", causal)
    compare_full(g, "bf16", causal, label=f"bf16 rect d={d} {nq}x{nk} causal={causal}")


def test_rect_decode_matches_noncausal():
    """One new query sees every cached key: causal and non-causal agree."""
    arrays = make_rect_inputs(4, 1, 700, 128, seed=32)
    a = run_gpu(arrays, "bf16", True)
    b = run_gpu(arrays, "bf16", False)
    compare_full(a, "bf16", True, label="bf16 decode 1x700 causal")
    for name in ("o", "lse", "dq", "dk", "dv"):
        scale = max(1.0, np.abs(b[name]).max())
        assert np.abs(a[name] - b[name]).max() <= 1e-2 * scale, name


def test_rect_rejects_causal_with_more_queries():
    arrays = make_rect_inputs(1, 65, 64, 64, seed=33)
    with pytest.raises(fa.FAError):
        run_gpu(arrays, "bf16", True)


# --------------------------------------------------------------------------- sliding window
# Causal attention restricted to each query's `window` most recent keys
# (window_attention_torch of "CS324 lecture 8, 03_online_softmax_and_flash.py").
# The windows cross tile edges at every offset: 1 (the diagonal alone), sizes
# below, at and above one tile, and windows wider than the sequence.
@pytest.mark.parametrize("window", [1, 7, 16, 37, 100, 199])
@pytest.mark.parametrize("tiles", [(16, 12), (64, 64), (32, 16)])
def test_window_fp32(window, tiles):
    arrays = make_inputs(2, 200, 32, seed=40)
    g = run_gpu(arrays, "fp32", True, tiles, tiles, tiles, window=window)
    compare_full(g, "fp32", True, label=f"fp32 window={window} n=200 tiles={tiles}", window=window)


@pytest.mark.parametrize("nq,nk,window", [(37, 100, 5), (37, 100, 70), (64, 200, 33), (1, 64, 10)])
def test_window_rect_fp32(nq, nk, window):
    arrays = make_rect_inputs(2, nq, nk, 32, seed=41)
    for tiles in ((16, 12), (64, 64)):
        g = run_gpu(arrays, "fp32", True, tiles, tiles, tiles, window=window)
        compare_full(g, "fp32", True, label=f"fp32 rect {nq}x{nk} window={window} tiles={tiles}",
                     window=window)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [1, 37, 64, 100, 257, 700])
@pytest.mark.parametrize("n", [333, 1000])
def test_window_bf16(d, window, n):
    arrays = make_inputs(2, n, d, seed=42)
    g = run_gpu(arrays, "bf16", True, window=window)
    compare_full(g, "bf16", True, label=f"bf16 d={d} n={n} window={window}", window=window)


@pytest.mark.parametrize("tiles", BF16_D128_TILINGS)
@pytest.mark.parametrize("window", [50, 300])
def test_window_bf16_tilings(tiles, window):
    arrays = make_inputs(2, 1000, 128, seed=43)
    g = run_gpu(arrays, "bf16", True, *tiles, window=window)
    compare_full(g, "bf16", True, label=f"bf16 window={window} tiles={tiles}", window=window)


@pytest.mark.parametrize("nq,nk,window", [(300, 1000, 128), (256, 4096, 1000), (1, 513, 100)])
@pytest.mark.parametrize("d", [64, 128])
def test_window_rect_bf16(nq, nk, window, d):
    arrays = make_rect_inputs(2, nq, nk, d, seed=44)
    g = run_gpu(arrays, "bf16", True, window=window)
    compare_full(g, "bf16", True, label=f"bf16 rect d={d} {nq}x{nk} window={window}", window=window)


def test_window_one_is_the_diagonal():
    """window = 1: each query sees only its own key, so P = 1 and O is that
    key's value row exactly; L is the scaled diagonal score."""
    arrays = make_inputs(2, 300, 128, seed=45)
    g = run_gpu(arrays, "bf16", True, window=1)
    assert np.array_equal(g["o"], g["v"])
    diag = np.einsum("hnd,hnd->hn", g["q"], g["k"]) / math.sqrt(128)
    assert np.abs(g["lse"] - diag).max() <= 1e-5 * max(1.0, np.abs(diag).max())
    assert np.array_equal(g["dv"], g["do"])


def test_window_covering_the_sequence_is_plain_causal():
    """A window of at least nk keys hides nothing: bitwise the causal result."""
    arrays = make_inputs(2, 500, 64, seed=46)
    a = run_gpu(arrays, "bf16", True)
    for window in (500, 501, 1 << 30):
        b = run_gpu(arrays, "bf16", True, window=window)
        for name in ("o", "lse", "dq", "dk", "dv"):
            assert np.array_equal(a[name], b[name]), (window, name)


def test_window_sampled_8192():
    """BH = 32, N = 8192, d = 128, bf16, causal with a 1024-key window, at the
    default tilings; sampled rows and columns against the oracle."""
    w = WORKLOADS["headline_8192_d128"]
    rng = np.random.default_rng(97)
    rows = np.unique(np.concatenate([[0, 1, 1023, 1024, 1025, 4095, 8191], rng.integers(0, w.n, 16)]))
    cols = np.unique(np.concatenate([[0, 1, 1024, 7167, 7168, 8191], rng.integers(0, w.n, 8)]))
    sampled_check(w, True, heads=[3], rows=rows, cols=cols, window=1024)


def test_window_rejects_bad_arguments():
    arrays = make_inputs(1, 64, 64, seed=47)
    with pytest.raises(fa.FAError):
        run_gpu(arrays, "bf16", False, window=16)
    with pytest.raises(fa.FAError):
        run_gpu(arrays, "bf16", True, window=-1)


# --------------------------------------------------------------------------- single-kernel backward
# fa_bwd_fused: dK, dV and dQ from one pass over the key tiles, dQ gathered
# with fp32 atomic adds (the design the two-kernel backward is weighed
# against).  Same oracle and tolerances as the two-kernel path.
def run_gpu_fused(arrays, dtype, causal, tiles=(0, 0), window=0, fwd_tiles=(0, 0)):
    q, k, v, do = cast_io(arrays, dtype, "cuda")
    o, lse = fa.forward(q, k, v, causal, None, *fwd_tiles, window=window)
    dq, dk, dv, delta = fa.backward_fused(q, k, v, o, do, lse, causal, None, tiles, window=window)
    torch.cuda.synchronize()
    return {name: to_f64(t) for name, t in
            dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta).items()}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [(16, 12), (64, 64), (32, 128)])
def test_fused_fp32(causal, tiles):
    arrays = make_inputs(2, 200, 32, seed=50)
    g = run_gpu_fused(arrays, "fp32", causal, tiles)
    compare_full(g, "fp32", causal, label=f"fused fp32 n=200 tiles={tiles} causal={causal}")


@pytest.mark.parametrize("nq,nk,causal,window", [(37, 100, True, 0), (200, 64, False, 0), (64, 200, True, 33),
                                                 (200, 200, True, 17)])
def test_fused_fp32_rect_and_window(nq, nk, causal, window):
    arrays = make_rect_inputs(2, nq, nk, 32, seed=51)
    g = run_gpu_fused(arrays, "fp32", causal, (16, 12), window=window)
    compare_full(g, "fp32", causal, label=f"fused fp32 {nq}x{nk} causal={causal} window={window}", window=window)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [100, 333, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_bf16(d, n, causal):
    arrays = make_inputs(2, n, d, seed=52)
    g = run_gpu_fused(arrays, "bf16", causal)
    compare_full(g, "bf16", causal, label=f"fused bf16 d={d} n={n} causal={causal}")
    # dK and dV come from the same arithmetic as fa_bwd_dkdv
    ref = run_gpu(arrays, "bf16", causal)
    for name in ("dk", "dv"):
        assert np.abs(g[name] - ref[name]).max() <= 1e-2 * max(1.0, np.abs(ref[name]).max()), name


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal,window", [(300, 1000, True, 0), (500, 200, False, 0),
                                                 (256, 4096, True, 1000), (1000, 1000, True, 100)])
def test_fused_bf16_rect_and_window(d, nq, nk, causal, window):
    arrays = make_rect_inputs(2, nq, nk, d, seed=53)
    g = run_gpu_fused(arrays, "bf16", causal, window=window)
    compare_full(g, "bf16", causal, label=f"fused bf16 d={d} {nq}x{nk} causal={causal} window={window}",
                 window=window)


def test_fused_sampled_8192():
    """BH = 32, N = 8192, d = 128, bf16, causal through the fused backward at
    the default tiling; sampled rows and columns against the oracle."""
    w = WORKLOADS["headline_8192_d128"]
    arrays = make_inputs(w.bh, w.n, w.d, seed=0)
    g = run_gpu_fused(arrays, w.dtype, True)
    rng = np.random.default_rng(96)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 4095, 8191], rng.integers(0, w.n, 16)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 8191], rng.integers(0, w.n, 8)]))
    tol = TOL[w.dtype]
    for h in (0, 17):
        q, k, v, do = (g[x][h] for x in ("q", "k", "v", "do"))
        dq_ref, _ = oracle.dq_rows(q, k, v, do, rows, causal=True)
        stats = oracle.head_row_stats(q, k, v, do, causal=True)
        dk_ref, dv_ref = oracle.dkdv_cols(q, k, v, do, cols, causal=True, stats=stats)
        rep = {
            "dq": np.abs(g["dq"][h][rows] - dq_ref).max() / np.abs(g["dq"][h]).max(),
            "dk": np.abs(g["dk"][h][cols] - dk_ref).max() / np.abs(g["dk"][h]).max(),
            "dv": np.abs(g["dv"][h][cols] - dv_ref).max() / np.abs(g["dv"][h]).max(),
        }
        _say(f"[fused 8192 head={h}] " + " ".join(f"{a}={b:.2e}" for a, b in rep.items()))
        for name in rep:
            assert rep[name] <= tol["grad"], (name, rep)
    for name in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(g[name])), name


def test_fused_workspace_contents_do_not_matter():
    """The call clears its workspace itself: garbage in it changes nothing
    beyond the order of the atomic adds."""
    arrays = make_inputs(2, 300, 128, seed=54)
    q, k, v, do = cast_io(arrays, "bf16", "cuda")
    o, lse = fa.forward(q, k, v, True)
    delta = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    fa.fa_bwd_preprocess(o, do, delta)
    outs = []
    for fill in (0.0, 1e30):
        ws = torch.full((fa.fa_bwd_fused_workspace_bytes(2, 300, 128, fa.FA_BF16) // 4,), fill,
                        dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fa.fa_bwd_fused(q, k, v, do, lse, delta, dq, dk, dv, ws, True)
        torch.cuda.synchronize()
        outs.append(to_f64(dq))
    scale = np.abs(outs[0]).max()
    assert np.abs(outs[0] - outs[1]).max() <= 1e-2 * scale
