"""The torch autograd drop-in (``flash_attention``) against the fp64 oracle and,
as a second referee, torch CPU autograd of the plain definition, in float64,
on seeded random inputs.

The loss is sum(O * W), so dO = W: the oracle's forward and backward
(``oracle.attention_forward`` / ``attention_backward``) give the expected O
and gradients directly; torch's reference is softmax(scale * Q K^T) V with
the end-aligned causal mask (and window), differentiated by torch on the CPU.
The inputs are the exact values of the device tensors (bf16 values upcast),
so input rounding is not charged to the kernels.  Tolerances are the parity
tests': float32 I/O: outputs 1e-5 absolute, gradients 1e-4 of the largest
reference gradient; bf16 I/O: outputs 1e-2, gradients 3e-2.
"""

import math
import sys

import pytest
import torch

import exact_tiled_attention_26_amd as fa
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-4), torch.bfloat16: (1e-2, 3e-2)}


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def reference_attention(q, k, v, causal, scale, window=0):
    """Causal masks are aligned to the end of the keys: query i sees keys
    0 .. i + nk - nq, and with a window only the last `window` of them."""
    s = scale * torch.matmul(q, k.transpose(-1, -2))
    if causal:
        nq, nk = q.shape[-2], k.shape[-2]
        hidden = torch.ones(nq, nk, dtype=torch.bool).triu(nk - nq + 1)
        if window:
            hidden |= torch.ones(nq, nk, dtype=torch.bool).tril(nk - nq - window)
        s = s.masked_fill(hidden, float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), v)


def _rel(err, ref):
    m = ref.abs().max().item()
    return err / (m if m > 0 else 1.0)


def _check_against_oracle(out, grads, q, k, v, w, causal, window, tol_o, tol_g):
    """O and (dQ, dK, dV) of the device call against the oracle on the same
    values, with dO = W (the gradient of sum(O * W))."""
    q, k, v, w = (t.detach().cpu().double().reshape(-1, *t.shape[-2:]).numpy() for t in (q, k, v, w))
    o_ref, _ = oracle.attention_forward(q, k, v, causal=causal, window=window)
    dq_ref, dk_ref, dv_ref, _ = oracle.attention_backward(q, k, v, w, causal=causal, window=window)
    err_o = abs(out.detach().cpu().double().reshape(o_ref.shape).numpy() - o_ref).max()
    assert err_o <= tol_o, ("oracle", "o", err_o)
    for name, a, b in (("dq", grads[0], dq_ref), ("dk", grads[1], dk_ref), ("dv", grads[2], dv_ref)):
        b = torch.from_numpy(b)
        err = _rel((a.cpu().double().reshape(b.shape) - b).abs().max().item(), b)
        assert err <= tol_g, ("oracle", name, err)


@pytest.mark.parametrize("dtype,shape,nk", [(torch.float32, (2, 3, 77, 32), 77),
                                            (torch.bfloat16, (2, 2, 300, 64), 300),
                                            (torch.float32, (2, 2, 50, 32), 130),
                                            (torch.bfloat16, (1, 3, 200, 128), 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_cpu_autograd(dtype, shape, nk, causal):
    _say(f"autograd dtype={dtype} q={shape} nk={nk} causal={causal}")
    g = torch.Generator().manual_seed(7)
    kshape = shape[:-2] + (nk, shape[-1])
    q, w = (torch.randn(shape, generator=g, dtype=torch.float64) for _ in range(2))
    k, v = (torch.randn(kshape, generator=g, dtype=torch.float64) for _ in range(2))
    qd, kd, vd = (t.to(dtype).cuda().requires_grad_(True) for t in (q, k, v))
    wd = w.to(dtype).cuda()
    out = fa.flash_attention(qd, kd, vd, causal=causal)
    (out.float() * wd.float()).sum().backward()
    torch.cuda.synchronize()

    qc, kc, vc = (t.detach().cpu().double().requires_grad_(True) for t in (qd, kd, vd))
    ref = reference_attention(qc, kc, vc, causal, 1.0 / math.sqrt(shape[-1]))
    (ref * wd.cpu().double()).sum().backward()

    tol_o, tol_g = TOL[dtype]
    _check_against_oracle(out, (qd.grad, kd.grad, vd.grad), qd, kd, vd, wd, causal, 0, tol_o, tol_g)
    assert out.shape == ref.shape == q.shape and out.dtype == dtype
    err_o = (out.detach().cpu().double() - ref.detach()).abs().max().item()
    assert err_o <= tol_o, err_o
    for name, a, b in (("dq", qd.grad, qc.grad), ("dk", kd.grad, kc.grad), ("dv", vd.grad, vc.grad)):
        assert a.dtype == dtype and a.shape == b.shape
        err = _rel((a.cpu().double() - b).abs().max().item(), b)
        assert err <= tol_g, (name, err)


@pytest.mark.parametrize("dtype,shape,nk,window", [(torch.float32, (2, 2, 90, 32), 90, 13),
                                                   (torch.bfloat16, (1, 2, 300, 128), 700, 200)])
def test_window_matches_cpu_autograd(dtype, shape, nk, window):
    _say(f"autograd window={window} dtype={dtype} q={shape} nk={nk}")
    g = torch.Generator().manual_seed(8)
    kshape = shape[:-2] + (nk, shape[-1])
    q, w = (torch.randn(shape, generator=g, dtype=torch.float64) for _ in range(2))
    k, v = (torch.randn(kshape, generator=g, dtype=torch.float64) for _ in range(2))
    qd, kd, vd = (t.to(dtype).cuda().requires_grad_(True) for t in (q, k, v))
    wd = w.to(dtype).cuda()
    out = fa.flash_attention(qd, kd, vd, causal=True, window=window)
    (out.float() * wd.float()).sum().backward()
    torch.cuda.synchronize()

    qc, kc, vc = (t.detach().cpu().double().requires_grad_(True) for t in (qd, kd, vd))
    ref = reference_attention(qc, kc, vc, True, 1.0 / math.sqrt(shape[-1]), window)
    (ref * wd.cpu().double()).sum().backward()

    tol_o, tol_g = TOL[dtype]
    _check_against_oracle(out, (qd.grad, kd.grad, vd.grad), qd, kd, vd, wd, True, window, tol_o, tol_g)
    err_o = (out.detach().cpu().double() - ref.detach()).abs().max().item()
    assert err_o <= tol_o, err_o
    for name, a, b in (("dq", qd.grad, qc.grad), ("dk", kd.grad, kc.grad), ("dv", vd.grad, vc.grad)):
        err = _rel((a.cpu().double() - b).abs().max().item(), b)
        assert err <= tol_g, (name, err)


def test_inside_a_model():
    """Gradients reach the projections around the op: a float32 block
    x -> qkv projection -> causal attention over 2 heads -> output projection,
    against the same block on the CPU in float64."""
    torch.manual_seed(3)
    bsz, n, c, heads = 2, 96, 64, 2
    d = c // heads
    x = torch.randn(bsz, n, c, dtype=torch.float64)
    w_qkv = torch.randn(c, 3 * c, dtype=torch.float64) / math.sqrt(c)
    w_o = torch.randn(c, c, dtype=torch.float64) / math.sqrt(c)

    def block(x, w_qkv, w_o, attn):
        qkv = (x @ w_qkv).view(bsz, n, 3, heads, d)
        q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))   # [bsz, heads, n, d], strided
        y = attn(q, k, v).transpose(1, 2).reshape(bsz, n, c)
        return ((y @ w_o) ** 2).mean()

    params_gpu = [t.float().cuda().requires_grad_(True) for t in (w_qkv, w_o)]
    loss_gpu = block(x.float().cuda(), *params_gpu, lambda q, k, v: fa.flash_attention(q, k, v, causal=True))
    loss_gpu.backward()
    torch.cuda.synchronize()

    params_cpu = [t.clone().requires_grad_(True) for t in (w_qkv, w_o)]
    loss_cpu = block(x, *params_cpu,
                     lambda q, k, v: reference_attention(q, k, v, True, 1.0 / math.sqrt(d)))
    loss_cpu.backward()

    assert abs(loss_gpu.item() - loss_cpu.item()) <= 1e-5 * abs(loss_cpu.item())
    for a, b in zip(params_gpu, params_cpu):
        err = _rel((a.grad.cpu().double() - b.grad).abs().max().item(), b.grad)
        assert err <= 1e-4, err


def test_explicit_scale_and_no_grad():
    q, k, v = (torch.randn(1, 64, 16, device="cuda") for _ in range(3))
    with torch.no_grad():
        out = fa.flash_attention(q, k, v, causal=False, scale=0.3)
    ref = reference_attention(q.cpu().double(), k.cpu().double(), v.cpu().double(), False, 0.3)
    assert (out.cpu().double() - ref).abs().max().item() <= 1e-5
