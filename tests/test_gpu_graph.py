"""The C ABI calls under HIP graph capture: the whole forward + backward
recorded once on torch's capture stream and replayed several times, with
eager work and synchronisations between the replays; every replay must
reproduce the eager results (bitwise for the deterministic two-kernel path,
within the atomic-order rounding for the single-kernel backward).  The
library only enqueues kernels on the stream it is given (no memsets, no
allocation, no synchronisation), so capture needs nothing special."""

import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_26_amd as fa
from workloads import cast_io, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _buffers(bh, n, d, seed, dtype="bf16"):
    q, k, v, do = cast_io(make_inputs(bh, n, d, seed=seed), dtype, "cuda")
    lse = torch.empty((bh, n), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    outs = dict(o=torch.empty_like(q), dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
    return q, k, v, do, lse, delta, outs


@pytest.mark.parametrize("dtype,fused", [("bf16", False), ("bf16", True), ("fp32", False), ("fp32", True)])
def test_graph_replays_match_eager(dtype, fused):
    _say(f"graph capture dtype={dtype} fused={fused}")
    bh, n, d = (4, 1000, 128) if dtype == "bf16" else (2, 300, 64)
    q, k, v, do, lse, delta, b = _buffers(bh, n, d, seed=60, dtype=dtype)
    ws = None
    nbytes = fa.fa_bwd_fused_workspace_bytes(bh, n, d, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32)
    if fused and nbytes:
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, b["o"], lse, True)
        fa.fa_bwd_preprocess(b["o"], do, delta)
        if fused:
            fa.fa_bwd_fused(q, k, v, do, lse, delta, b["dq"], b["dk"], b["dv"], ws, True)
        else:
            fa.fa_bwd_dkdv(q, k, v, do, lse, delta, b["dk"], b["dv"], True)
            fa.fa_bwd_dq(q, k, v, do, lse, delta, b["dq"], True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm up off the default stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {name: to_f64(t) for name, t in dict(lse=lse, delta=delta, **b).items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for replay in range(3):
        for t in (lse, delta, *b.values()):
            t.fill_(float("nan"))   # eager work between replays; the replay must overwrite it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in dict(lse=lse, delta=delta, **b).items():
            got = to_f64(t)
            if fused and name == "dq":
                scale = np.abs(eager[name]).max()
                tol = 1e-2 if dtype == "bf16" else 1e-5
                assert np.abs(got - eager[name]).max() <= tol * scale, (replay, name)
            else:
                assert np.array_equal(got, eager[name]), (replay, name)
