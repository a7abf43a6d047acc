"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the passage it follows.  Together they are chosen so that a
plausible mistake in the oracle (a dropped scale, a wrong sign, a transposed
operand, a wrong mask direction, a wrong logsumexp) fails at least one of
them; ``test_pins_catch_planted_mistakes`` demonstrates that for a few such
mistakes planted in copies of the oracle's outputs.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as A
from oracle import tiled as T
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- online softmax
def test_online_softmax_worked_example():
    """CS324 lecture 8, demo2_online: x read 3 at a time."""
    g = _golden("online_softmax_trace.json")
    x = np.array(g["x"])
    out, steps = oracle.online_softmax(x, g["block"], trace=True)
    assert [s[0] for s in steps] == g["entries_read_after_each_block"]
    assert [s[1] for s in steps] == g["running_max_after_each_block"]
    # closed form of the running denominator: after reading the first e
    # entries with running max m, l = sum_{i<e} exp(x_i - m)
    for e, m, l in steps:
        expect = sum(math.exp(xi - m) for xi in g["x"][:e])
        assert abs(l - expect) <= 1e-15 * expect
    # the page's final identity: l = sum exp(x - 6)
    assert abs(steps[-1][2] - sum(math.exp(xi - 6.0) for xi in g["x"])) < 1e-15
    np.testing.assert_allclose(out, scipy.special.softmax(x), rtol=1e-15, atol=0)


def test_online_softmax_block_sizes_agree():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(37) * 20
    ref = scipy.special.softmax(x)
    for b in (1, 2, 3, 7, 36, 37, 100):
        np.testing.assert_allclose(oracle.online_softmax(x, b), ref, rtol=1e-13, atol=0)


def test_online_softmax_no_overflow():
    """CS324 lecture 8, demo1_overflow: x = [1000, 1001, 1002] overflows the
    unshifted formula; the max-subtracted one does not."""
    x = np.array([1000.0, 1001.0, 1002.0])
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(x) / np.exp(x).sum()
    assert not np.all(np.isfinite(naive))
    out = oracle.online_softmax(x, 2)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, scipy.special.softmax(x), rtol=1e-14)


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences(causal):
    """CS349E lecture 11, demo1_gradcheck protocol: default_rng(0); Q, K, V, G
    drawn in that order, each 48 x 16; loss = sum(O * G); central differences
    with eps = 1e-6 at 6 random entries each of Q, K and V (indices drawn from
    the same generator after the inputs).  The page reports errors of order
    1e-9; the bound here is 1e-7."""
    rng = np.random.default_rng(0)
    n, d = 48, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    g = rng.standard_normal((n, d))
    # the page runs the non-causal pass first, drawing indices as it goes
    if causal:
        for _ in range(18):
            rng.integers(n), rng.integers(d)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, g, causal=causal)
    grads = {"Q": dq, "K": dk, "V": dv}
    eps = 1e-6
    worst = 0.0
    for name in ("Q", "K", "V"):
        for _ in range(6):
            r, c = int(rng.integers(n)), int(rng.integers(d))
            args_p = {"Q": q.copy(), "K": k.copy(), "V": v.copy()}
            args_m = {"Q": q.copy(), "K": k.copy(), "V": v.copy()}
            args_p[name][r, c] += eps
            args_m[name][r, c] -= eps
            fp = np.sum(oracle.attention_forward(args_p["Q"], args_p["K"], args_p["V"], causal=causal)[0] * g)
            fm = np.sum(oracle.attention_forward(args_m["Q"], args_m["K"], args_m["V"], causal=causal)[0] * g)
            worst = max(worst, abs((fp - fm) / (2 * eps) - grads[name][r, c]))
    assert worst < 1e-7, worst


def test_full_gradient_matches_central_differences_small():
    """All entries of dQ, dK, dV on a tiny causal case (N=5, d=3)."""
    rng = np.random.default_rng(11)
    q, k, v, g = (rng.standard_normal((5, 3)) for _ in range(4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, g, causal=True)
    eps = 1e-6
    for x, gx in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            sub = lambda t: [t if y is x else y for y in (q, k, v)]  # noqa: E731
            fp = np.sum(oracle.attention_forward(*sub(xp), causal=True)[0] * g)
            fm = np.sum(oracle.attention_forward(*sub(xm), causal=True)[0] * g)
            assert abs((fp - fm) / (2 * eps) - gx[idx]) < 1e-8


# ---------------------------------------------------------------- library referees
def _torch_reference(q, k, v, do, causal, scale):
    """CS324 lecture 8, demo4_backward: standard attention as torch CPU fp64
    ops (causal via a lower-triangular mask), differentiated by autograd."""
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(128, 16), (97, 8), (1, 4)])
def test_matches_torch_autograd(causal, n, d):
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, causal=causal)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=causal)
    ro, rdq, rdk, rdv = _torch_reference(q, k, v, do, causal, scale)
    for a, b in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))
    # L against scipy's logsumexp of the masked scores
    s = scale * q @ k.T
    if causal:
        s[np.triu_indices(n, 1)] = -np.inf
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_explicit_scale_reaches_both_gradients():
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((40, 8)) for _ in range(4))
    for causal in (False, True):
        o, _ = oracle.attention_forward(q, k, v, scale=0.3, causal=causal)
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale=0.3, causal=causal)
        ro, rdq, rdk, rdv = _torch_reference(q, k, v, do, causal, 0.3)
        for a, b in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- D identity
@pytest.mark.parametrize("causal", [False, True])
def test_delta_identity(causal):
    """CS336 Assignment 2 notes 1.4 Eq 17: sum_j P_ij dP_ij = sum_k dO_ik O_ik."""
    q, k, v, do = (a[0] for a in make_inputs(1, 200, 24, seed=7))
    o, _ = oracle.attention_forward(q, k, v, causal=causal)
    *_, delta = oracle.attention_backward(q, k, v, do, causal=causal)
    ident = oracle.delta_from_output(o, do)
    np.testing.assert_allclose(delta, ident, rtol=0, atol=1e-12 * np.abs(ident).max())


# ---------------------------------------------------------------- tiled model
SWEEP = [(16, 16), (32, 64), (64, 32), (128, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", SWEEP)
def test_tiled_equals_definition_block_sweep(causal, br, bc):
    """CS324 lecture 8, demo3_forward: N = 256, d = 32, blocks (16,16),
    (32,64), (64,32), (128,128); the tiled result equals standard attention to
    fp64 rounding (the page reports ~1e-16)."""
    q, k, v, do = (a[0] for a in make_inputs(1, 256, 32, seed=0))
    o, lse = oracle.attention_forward(q, k, v, causal=causal)
    to, tl, _ = oracle.tiled_forward(q, k, v, br, bc, causal=causal)
    assert np.abs(to - o).max() <= 1e-13 * np.abs(o).max()
    assert np.abs(tl - lse).max() <= 1e-13 * np.abs(lse).max()
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, causal=causal)
    tdq, tdk, tdv, tdelta, *_ = oracle.tiled_backward(q, k, v, to, do, tl, br, bc, causal=causal)
    for a, b in ((tdq, dq), (tdk, dk), (tdv, dv), (tdelta, delta)):
        assert np.abs(a - b).max() <= 1e-13 * np.abs(b).max()


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_definition_16x12(causal):
    """CS349E lecture 11, demo1_gradcheck: N = 48, d = 16, blocks 16 x 12."""
    q, k, v, do = (a[0] for a in make_inputs(1, 48, 16, seed=0))
    o, lse = oracle.attention_forward(q, k, v, causal=causal)
    to, tl, _ = oracle.tiled_forward(q, k, v, 16, 12, causal=causal)
    np.testing.assert_allclose(to, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(tl, lse, rtol=0, atol=1e-14)
    g = oracle.attention_backward(q, k, v, do, causal=causal)
    tg = oracle.tiled_backward(q, k, v, to, do, tl, 16, 12, causal=causal)
    for a, b in zip(tg[:4], g):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_tiled_ragged_last_tile():
    """CS324 lecture 8, flash_attention_torch: when N is not a multiple of the
    block the last block is smaller."""
    q, k, v, do = (a[0] for a in make_inputs(1, 50, 8, seed=2))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal=causal)
        to, tl, _ = oracle.tiled_forward(q, k, v, 16, 12, causal=causal)
        np.testing.assert_allclose(to, o, rtol=0, atol=1e-14)
        tg = oracle.tiled_backward(q, k, v, to, do, tl, 32, 16, causal=causal)
        g = oracle.attention_backward(q, k, v, do, causal=causal)
        for a, b in zip(tg[:4], g):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_causal_tile_fraction():
    """CS349E lecture 11, demo4_causal: with T = N/B square tiles per side the
    causal skip computes T(T+1)/2 tiles, a fraction 1/2 + 1/(2T)."""
    g = _golden("causal_tile_fraction.json")
    n = g["n"]
    for b in g["square_blocks"]:
        t = n // b
        got = oracle.causal_tiles_computed(n, b, b)
        assert got == t * (t + 1) // 2
        assert abs(got / t**2 - (0.5 + 0.5 / t)) < 1e-15
    # non-square: brute force over elements -- a tile is needed iff some key in
    # it is visible to some query in it
    for br, bc in g["non_square_blocks"]:
        rows = np.arange(n)
        need = 0
        for i0 in range(0, n, br):
            last_row = rows[i0:i0 + br].max()
            for j0 in range(0, n, bc):
                need += int(j0 <= last_row)
        assert oracle.causal_tiles_computed(n, br, bc) == need
    # the tiled forward counts the same tiles (small size, element brute force)
    q, k, v, _ = (a[0] for a in make_inputs(1, 96, 4, seed=1))
    for br, bc in ((16, 16), (32, 16), (16, 32), (24, 40)):
        _, _, cnt = oracle.tiled_forward(q, k, v, br, bc, causal=True)
        brute = sum(
            int(np.any(np.arange(j0, min(96, j0 + bc))[None, :] <= np.arange(i0, min(96, i0 + br))[:, None]))
            for i0 in range(0, 96, br) for j0 in range(0, 96, bc))
        assert cnt == brute == oracle.causal_tiles_computed(96, br, bc)


# ---------------------------------------------------------------- closed forms
def test_special_case_constant_v():
    """Rows of P sum to one, so V = 1 gives O = 1 (CS336 notes 1.1)."""
    q, k, _, _ = (a[0] for a in make_inputs(1, 64, 8, seed=9))
    for causal in (False, True):
        o, _ = oracle.attention_forward(q, k, np.ones((64, 8)), causal=causal)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_special_case_equal_keys():
    """All keys equal: P is uniform over the visible keys, O is the (prefix)
    mean of V, L_i = scale q_i.k + ln(#visible) and dQ = 0."""
    rng = np.random.default_rng(10)
    n, d = 30, 6
    q, v, do = (rng.standard_normal((n, d)) for _ in range(3))
    kr = rng.standard_normal(d)
    k = np.tile(kr, (n, 1))
    s = 1 / math.sqrt(d)
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal=causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.tile(v.mean(0), (n, 1))
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, s * q @ kr + np.log(cnt), rtol=0, atol=1e-13)
        dq, *_ = oracle.attention_backward(q, k, v, do, causal=causal)
        np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)


def test_special_case_single_token():
    """N = 1: O = V, L = scale q.k, dV = dO, dQ = dK = 0."""
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal((1, 5)) for _ in range(4))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal=causal)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, (q @ k.T)[0] / math.sqrt(5), rtol=0, atol=1e-15)
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=causal)
        np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dq, 0, atol=1e-15)
        np.testing.assert_allclose(dk, 0, atol=1e-15)


def test_key_shift_invariance():
    """K <- K + 1 c^T shifts each row's scores by scale q_i.c: L shifts by
    that amount and O, dQ, dK, dV are unchanged."""
    rng = np.random.default_rng(13)
    q, k, v, do = (rng.standard_normal((40, 8)) for _ in range(4))
    c = rng.standard_normal(8)
    s = 1 / math.sqrt(8)
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, causal=causal)
        o2, l2 = oracle.attention_forward(q, k + c, v, causal=causal)
        np.testing.assert_allclose(o2, o1, atol=1e-13)
        np.testing.assert_allclose(l2, l1 + s * q @ c, atol=1e-13)
        g1 = oracle.attention_backward(q, k, v, do, causal=causal)
        g2 = oracle.attention_backward(q, k + c, v, do, causal=causal)
        for a, b in zip(g1[:3], g2[:3]):
            np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """From Eq 15-19 and sum_j P_ij = 1: sum_j dV_j = sum_i dO_i and
    sum_j dK_j = 0 (rows of dS sum to zero)."""
    q, k, v, do = (a[0] for a in make_inputs(1, 120, 16, seed=14))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=causal)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)


def test_large_scores_stay_finite():
    """Scores of order 1e3 (Q scaled by 50): the max-subtracted softmax stays
    finite (CS324 lecture 8, demo1_overflow) and matches torch fp64."""
    q, k, v, do = (a[0] for a in make_inputs(1, 64, 16, seed=15))
    q = q * 50
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal=causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=causal)
        ro, rdq, rdk, rdv = _torch_reference(q, k, v, do, causal, 0.25)
        np.testing.assert_allclose(o, ro, atol=1e-12)
        for a, b in ((dq, rdq), (dk, rdk), (dv, rdv)):
            np.testing.assert_allclose(a, b, atol=1e-10 * max(1, np.abs(b).max()))


# ---------------------------------------------------------------- sampled outputs
@pytest.mark.parametrize("causal", [False, True])
def test_sampled_outputs_match_full(causal):
    q, k, v, do = (a[0] for a in make_inputs(1, 300, 16, seed=16))
    o, lse = oracle.attention_forward(q, k, v, causal=causal, chunk=64)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, causal=causal, chunk=77)
    rows = np.array([0, 1, 63, 150, 299])
    ro, rl = oracle.forward_rows(q, k, v, rows, causal=causal)
    np.testing.assert_allclose(ro, o[rows], atol=1e-14)
    np.testing.assert_allclose(rl, lse[rows], atol=1e-14)
    rdq, rdelta = oracle.dq_rows(q, k, v, do, rows, causal=causal)
    np.testing.assert_allclose(rdq, dq[rows], atol=1e-13)
    np.testing.assert_allclose(rdelta, delta[rows], atol=1e-13)
    cols = np.array([0, 5, 200, 299])
    ck, cv = oracle.dkdv_cols(q, k, v, do, cols, causal=causal, chunk=50)
    np.testing.assert_allclose(ck, dk[cols], atol=1e-13)
    np.testing.assert_allclose(cv, dv[cols], atol=1e-13)
    # chunking only regroups sums
    o2, l2 = oracle.attention_forward(q, k, v, causal=causal, chunk=1000)
    np.testing.assert_allclose(o2, o, atol=1e-15)


def test_batched_equals_per_head():
    q, k, v, do = make_inputs(3, 40, 8, seed=17)
    o, lse = oracle.attention_forward(q, k, v, causal=True)
    g = oracle.attention_backward(q, k, v, do, causal=True)
    for h in range(3):
        oh, lh = oracle.attention_forward(q[h], k[h], v[h], causal=True)
        np.testing.assert_array_equal(o[h], oh)
        gh = oracle.attention_backward(q[h], k[h], v[h], do[h], causal=True)
        for a, b in zip(g, gh):
            np.testing.assert_array_equal(a[h], b)


# ---------------------------------------------------------------- pin power
def test_pins_catch_planted_mistakes():
    """Plausible oracle mistakes, planted in copies of its outputs, fail the
    library referee (torch autograd) by a wide margin."""
    rng = np.random.default_rng(18)
    n, d = 32, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    ro, rdq, rdk, rdv = _torch_reference(q, k, v, do, True, 1 / math.sqrt(d))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=True)
    planted = {
        "dK without scale": (dk * math.sqrt(d), rdk),
        "dS sign flipped (dQ)": (-dq, rdq),
        "dV from P instead of P^T": (
            np.exp(A._scores(q, k, 1 / math.sqrt(d), True, np.arange(n)) -
                   oracle.attention_forward(q, k, v, causal=True)[1][:, None]) @ do, rdv),
    }
    for name, (bad, ref) in planted.items():
        assert np.abs(bad - ref).max() > 1e-3, name
    # a mask in the wrong direction changes the forward
    o_up, _ = oracle.attention_forward(q[::-1], k[::-1], v[::-1], causal=True)
    assert np.abs(o_up[::-1] - ro).max() > 1e-3


# --------------------------------------------------------------------------
# Queries and keys of different lengths (causal mask aligned to the end of
# the keys: query i sees keys 0 .. i + N_k - N_q)
# --------------------------------------------------------------------------

def _torch_rect_reference(q, k, v, do, causal, scale):
    """torch SDPA on the CPU in float64 with an explicit boolean mask (True =
    the key takes part) built from the end-aligned rule."""
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    mask = None
    if causal:
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        mask = j <= i + (nk - nq)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], attn_mask=mask, scale=scale)[0, 0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# (causal with more queries than keys is rejected by the oracle: test below)
@pytest.mark.parametrize("causal,nq,nk", [(c, nq, nk) for nq, nk in ((37, 100), (1, 64), (64, 64), (90, 31))
                                          for c in (False, True) if not (c and nq > nk)])
def test_rect_matches_torch_sdpa_mask(causal, nq, nk):
    rng = np.random.default_rng(21)
    d = 8
    q, do = (rng.standard_normal((nq, d)) for _ in range(2))
    k, v = (rng.standard_normal((nk, d)) for _ in range(2))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, causal=causal, chunk=16)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, causal=causal, chunk=16)
    ro, rdq, rdk, rdv = _torch_rect_reference(q, k, v, do, causal, scale)
    for a, b in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))
    np.testing.assert_allclose(delta, oracle.delta_from_output(o, do), atol=1e-12)


def test_rect_causal_is_the_tail_of_square_attention():
    """N_q queries against N_k keys, causal, equal the last N_q rows of square
    causal attention over N_k queries whose last N_q rows are those queries;
    with dO zero on the other rows, dK and dV are the square ones as well."""
    rng = np.random.default_rng(22)
    nk, nq, d = 120, 45, 16
    q_full, k, v, do_full = (rng.standard_normal((nk, d)) for _ in range(4))
    do_full[: nk - nq] = 0.0
    o_sq, l_sq = oracle.attention_forward(q_full, k, v, causal=True)
    dq_sq, dk_sq, dv_sq, _ = oracle.attention_backward(q_full, k, v, do_full, causal=True)
    q, do = q_full[nk - nq:], do_full[nk - nq:]
    o, lse = oracle.attention_forward(q, k, v, causal=True)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=True)
    np.testing.assert_allclose(o, o_sq[nk - nq:], atol=1e-14)
    np.testing.assert_allclose(lse, l_sq[nk - nq:], atol=1e-13)
    np.testing.assert_allclose(dq, dq_sq[nk - nq:], atol=1e-13)
    np.testing.assert_allclose(dk, dk_sq, atol=1e-13)
    np.testing.assert_allclose(dv, dv_sq, atol=1e-13)


def test_rect_decode_sees_every_key():
    """One new query (decode) sees every cached key ([CS349E-L11]
    demo4_causal observations), so causal and non-causal agree."""
    rng = np.random.default_rng(23)
    q, do = (rng.standard_normal((1, 32)) for _ in range(2))
    k, v = (rng.standard_normal((200, 32)) for _ in range(2))
    a = oracle.attention_forward(q, k, v, causal=True)
    b = oracle.attention_forward(q, k, v, causal=False)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)
    ga = oracle.attention_backward(q, k, v, do, causal=True)
    gb = oracle.attention_backward(q, k, v, do, causal=False)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, atol=1e-15)


def test_rect_causal_needs_enough_keys():
    rng = np.random.default_rng(24)
    q = rng.standard_normal((10, 4))
    k = rng.standard_normal((9, 4))
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, k, causal=True)
    rows = oracle.attention_forward(q, k, k, causal=False)[0]
    assert rows.shape == (10, 4)


def test_rect_sampled_outputs_match_full():
    q, do = (a[0] for a in make_inputs(1, 70, 16, seed=25)[:2])
    k, v = (a[0] for a in make_inputs(1, 150, 16, seed=26)[:2])
    o, lse = oracle.attention_forward(q, k, v, causal=True)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=True)
    rows, cols = np.array([0, 33, 69]), np.array([0, 80, 149])
    ro, rl = oracle.forward_rows(q, k, v, rows, causal=True)
    np.testing.assert_allclose(ro, o[rows], atol=1e-14)
    np.testing.assert_allclose(oracle.dq_rows(q, k, v, do, rows, causal=True)[0], dq[rows], atol=1e-13)
    ck, cv = oracle.dkdv_cols(q, k, v, do, cols, causal=True)
    np.testing.assert_allclose(ck, dk[cols], atol=1e-13)
    np.testing.assert_allclose(cv, dv[cols], atol=1e-13)


def test_rect_pins_catch_a_top_left_mask(monkeypatch):
    """Aligning the rectangular causal mask to the start of the keys (offset
    0) instead of their end is a plausible mistake; the torch reference with
    the explicit end-aligned mask rejects it."""
    rng = np.random.default_rng(27)
    nq, nk, d = 20, 50, 8
    q, do = (rng.standard_normal((nq, d)) for _ in range(2))
    k, v = (rng.standard_normal((nk, d)) for _ in range(2))
    ro = _torch_rect_reference(q, k, v, do, True, 1 / math.sqrt(d))[0]
    monkeypatch.setattr(A, "_causal_offset", lambda nq_, nk_, causal: 0)
    bad, _ = oracle.attention_forward(q, k, v, causal=True)
    assert np.abs(bad - ro).max() > 1e-2


# --------------------------------------------------------------------------
# Sliding window ([CS324-L8] window_attention_torch): with causal masking a
# query sees only its `window` most recent keys
# --------------------------------------------------------------------------

def _torch_band_reference(q, k, v, do, window, scale):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    i = torch.arange(nq)[:, None] + (nk - nq)
    j = torch.arange(nk)[None, :]
    mask = (j <= i) & (j > i - window)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], attn_mask=mask, scale=scale)[0, 0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("nq,nk,window", [(64, 64, 5), (64, 64, 16), (30, 100, 7), (1, 50, 10), (50, 50, 200)])
def test_window_matches_torch_sdpa_band(nq, nk, window):
    rng = np.random.default_rng(40)
    d = 8
    q, do = (rng.standard_normal((nq, d)) for _ in range(2))
    k, v = (rng.standard_normal((nk, d)) for _ in range(2))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, causal=True, window=window, chunk=16)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, causal=True, window=window, chunk=16)
    ro, rdq, rdk, rdv = _torch_band_reference(q, k, v, do, window, scale)
    for a, b in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))
    np.testing.assert_allclose(delta, oracle.delta_from_output(o, do), atol=1e-12)


def test_window_special_cases():
    """window = 1: each query sees only its own position, so O_i = V_{i+off},
    L_i = S_{i,i+off}, dV_j = dO_{j-off}, and dS = P (dP - D) = 0 gives
    dQ = dK = 0.  window >= N_k: plain causal attention."""
    rng = np.random.default_rng(41)
    nq, nk, d = 20, 35, 8
    q, do = (rng.standard_normal((nq, d)) for _ in range(2))
    k, v = (rng.standard_normal((nk, d)) for _ in range(2))
    off = nk - nq
    o, lse = oracle.attention_forward(q, k, v, causal=True, window=1)
    np.testing.assert_allclose(o, v[off:], atol=1e-15)
    np.testing.assert_allclose(lse, (q * k[off:]).sum(axis=1) / math.sqrt(d), atol=1e-13)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=True, window=1)
    np.testing.assert_allclose(dv[off:], do, atol=1e-15)
    assert np.abs(dv[:off]).max() == 0.0
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    full = oracle.attention_forward(q, k, v, causal=True)
    wide = oracle.attention_forward(q, k, v, causal=True, window=nk)
    np.testing.assert_allclose(wide[0], full[0], atol=0)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v, causal=False, window=4)
    with pytest.raises(ValueError):
        oracle.attention_forward(q, k, v, causal=True, window=-1)


def test_window_sampled_outputs_match_full():
    q, k, v, do = (a[0] for a in make_inputs(1, 200, 16, seed=42))
    o, lse = oracle.attention_forward(q, k, v, causal=True, window=37)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, causal=True, window=37)
    rows, cols = np.array([0, 36, 37, 199]), np.array([0, 100, 199])
    np.testing.assert_allclose(oracle.forward_rows(q, k, v, rows, causal=True, window=37)[0], o[rows], atol=1e-14)
    np.testing.assert_allclose(oracle.dq_rows(q, k, v, do, rows, causal=True, window=37)[0], dq[rows], atol=1e-13)
    ck, cv = oracle.dkdv_cols(q, k, v, do, cols, causal=True, window=37)
    np.testing.assert_allclose(ck, dk[cols], atol=1e-13)
    np.testing.assert_allclose(cv, dv[cols], atol=1e-13)
