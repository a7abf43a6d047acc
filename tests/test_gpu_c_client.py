"""The plain C client of the ABI (tests/c_abi/fa_c_client.c, no Python or
torch in the process) on the GPU: its forward and backward must equal the
binding's bit for bit (same kernels, same default tilings) and match the
oracle within the bf16 tolerances of the parity tests."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_26_amd as fa
import oracle
from exact_tiled_attention_26_amd.build import C_CLIENT
from workloads import cast_io, make_inputs, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bh,n,d,causal,window,fused", [(2, 333, 128, 1, 0, 0), (3, 200, 64, 0, 0, 0),
                                                        (2, 500, 128, 1, 77, 0), (2, 300, 64, 1, 0, 1)])
def test_c_client_matches_binding_and_oracle(tmp_path, bh, n, d, causal, window, fused):
    print(f"C client bh={bh} n={n} d={d} causal={causal} window={window} fused={fused}", file=sys.stderr, flush=True)
    assert os.path.exists(C_CLIENT), "build the C client first (__graft_entry__.build())"
    q, k, v, do = cast_io(make_inputs(bh, n, d, seed=70), "bf16", "cpu")
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        for t in (q, k, v, do):
            f.write(t.contiguous().view(torch.int16).numpy().tobytes())
    r = subprocess.run([C_CLIENT, str(inp), str(out), str(bh), str(n), str(d), str(causal), str(window), str(fused)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    raw = np.fromfile(out, dtype=np.uint8)
    te, re_ = bh * n * d * 2, bh * n * 4
    parts, pos = {}, 0
    for name, nbytes, dt in (("o", te, torch.bfloat16), ("lse", re_, torch.float32), ("dq", te, torch.bfloat16),
                             ("dk", te, torch.bfloat16), ("dv", te, torch.bfloat16), ("delta", re_, torch.float32)):
        buf = torch.from_numpy(raw[pos:pos + nbytes].copy())
        parts[name] = buf.view(dt).reshape((bh, n, d) if dt == torch.bfloat16 else (bh, n))
        pos += nbytes
    assert pos == raw.size

    # the binding on the same inputs: identical bits (the fused backward's dQ
    # depends on the order of its atomic adds, so it is compared with a
    # tolerance instead)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, bool(causal), window=window)
    if fused:
        dq, dk, dv, delta = fa.backward_fused(qd, kd, vd, o, dod, lse, bool(causal), window=window)
    else:
        dq, dk, dv, delta = fa.backward(qd, kd, vd, o, dod, lse, bool(causal), window=window)
    torch.cuda.synchronize()
    for name, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta).items():
        if fused and name == "dq":
            ref = t.cpu().double()
            assert (parts[name].double() - ref).abs().max() <= 1e-2 * ref.abs().max(), name
        else:
            assert torch.equal(parts[name], t.cpu()), name

    # and the oracle
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o_ref, l_ref = oracle.attention_forward(q64, k64, v64, causal=bool(causal), window=window)
    g_ref = oracle.attention_backward(q64, k64, v64, do64, causal=bool(causal), window=window)
    assert np.abs(to_f64(parts["o"]) - o_ref).max() <= 1e-2
    assert np.abs(to_f64(parts["lse"]) - l_ref).max() <= 1e-3
    for name, ref in zip(("dq", "dk", "dv"), g_ref):
        assert np.abs(to_f64(parts[name]) - ref).max() <= 3e-2 * np.abs(ref).max(), name
