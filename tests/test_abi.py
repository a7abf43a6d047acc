"""C-ABI tests that need no GPU: libfa.so loads, exports every function that
include/fa.h declares, and rejects invalid arguments on the host before any
HIP call (so nothing is launched)."""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_26_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x10000      # 16-byte aligned fake addresses (never dereferenced: calls are rejected first)
B = 0x20000
C = 0x30000
D_ = 0x40000
E = 0x50000
F = 0x60000
G = 0x70000
H = 0x80000


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\**\s*(fa_[a-z0-9_]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert names == sorted(fa.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name
    # also check the dynamic symbol table directly
    so = ctypes.CDLL(fa.LIB_PATH)
    for name in names:
        assert ctypes.cast(getattr(so, name), ctypes.c_void_p).value


def test_version_and_strings(lib):
    assert fa.fa_abi_version() == 5
    for code in range(6):
        assert fa.fa_status_str(code)
    assert fa.fa_status_str(99) == "unknown status"


def test_default_tiles(lib):
    assert fa.fa_default_tiles(fa.FA_BF16, 128, fa.KERNEL_FWD) == (256, 64)
    assert fa.fa_default_tiles(fa.FA_BF16, 128, fa.KERNEL_DKDV) == (128, 128)
    assert fa.fa_default_tiles(fa.FA_BF16, 64, fa.KERNEL_DKDV) == (128, 128)
    assert fa.fa_default_tiles(fa.FA_BF16, 128, fa.KERNEL_DQ) == (256, 32)
    assert fa.fa_default_tiles(fa.FA_F32, 16, fa.KERNEL_FWD) == (128, 64)
    assert fa.fa_default_tiles(fa.FA_F32, 64, fa.KERNEL_DKDV) == (64, 64)
    assert fa.fa_default_tiles(fa.FA_F32, 128, fa.KERNEL_DQ) == (128, 64)
    with pytest.raises(fa.FAError):
        fa.fa_default_tiles(fa.FA_BF16, 16, fa.KERNEL_FWD)
    with pytest.raises(fa.FAError):
        fa.fa_default_tiles(fa.FA_F32, 48, fa.KERNEL_FWD)
    bm = ctypes.c_int()
    assert lib.fa_default_tiles(0, 64, 7, ctypes.byref(bm), ctypes.byref(bm)) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_default_tiles(0, 64, 0, None, None) == fa.FA_ERR_INVALID_ARG


def fwd(lib, q=A, k=B, v=C, o=D_, lse=E, bh=1, n=64, d=64, dtype=fa.FA_BF16, scale=0.125, causal=1,
        bm=0, bn=0):
    return lib.fa_fwd(q, k, v, o, lse, bh, n, d, dtype, scale, causal, bm, bn, None)


def dkdv(lib, **kw):
    a = dict(q=A, k=B, v=C, dO=D_, lse=E, delta=F, dk=G, dv=H, bh=1, n=64, d=64, dtype=fa.FA_BF16,
             scale=0.125, causal=1, bm=0, bn=0)
    a.update(kw)
    return lib.fa_bwd_dkdv(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dk"], a["dv"],
                           a["bh"], a["n"], a["d"], a["dtype"], a["scale"], a["causal"], a["bm"], a["bn"], None)


def dq(lib, **kw):
    a = dict(q=A, k=B, v=C, dO=D_, lse=E, delta=F, dq=G, bh=1, n=64, d=64, dtype=fa.FA_BF16,
             scale=0.125, causal=1, bm=0, bn=0)
    a.update(kw)
    return lib.fa_bwd_dq(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dq"],
                         a["bh"], a["n"], a["d"], a["dtype"], a["scale"], a["causal"], a["bm"], a["bn"], None)


def test_null_pointers_rejected(lib):
    assert fwd(lib, q=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, lse=0) == fa.FA_ERR_INVALID_ARG
    assert dkdv(lib, delta=0) == fa.FA_ERR_INVALID_ARG
    assert dq(lib, dq=0) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_preprocess(A, 0, C, 1, 64, 64, fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG


def test_misaligned_rejected(lib):
    assert fwd(lib, k=B + 2) == fa.FA_ERR_MISALIGNED
    assert fwd(lib, lse=E + 4) == fa.FA_ERR_MISALIGNED
    assert dkdv(lib, dv=H + 8) == fa.FA_ERR_MISALIGNED
    assert dq(lib, dO=D_ + 2) == fa.FA_ERR_MISALIGNED
    assert lib.fa_bwd_preprocess(A + 2, B, C, 1, 64, 64, fa.FA_BF16, None) == fa.FA_ERR_MISALIGNED


def test_sizes_and_dtypes(lib):
    assert fwd(lib, n=-1) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, bh=-3) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, d=0) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, dtype=7) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, d=48) == fa.FA_ERR_UNSUPPORTED
    assert fwd(lib, d=16, dtype=fa.FA_BF16) == fa.FA_ERR_UNSUPPORTED   # bf16 provides d = 64, 128
    assert fwd(lib, n=(1 << 24) + 1) == fa.FA_ERR_UNSUPPORTED
    assert fwd(lib, bh=(1 << 20) + 1) == fa.FA_ERR_UNSUPPORTED
    assert dkdv(lib, d=256) == fa.FA_ERR_UNSUPPORTED
    assert dq(lib, d=32, dtype=fa.FA_BF16) == fa.FA_ERR_UNSUPPORTED


def test_grid_limit(lib):
    # float32 dK/dV with 4-key tiles at the largest n and bh would exceed 2^31 workgroups
    assert dkdv(lib, dtype=fa.FA_F32, d=16, bm=16, bn=4, n=1 << 24, bh=1 << 10) == fa.FA_ERR_UNSUPPORTED


def test_scale_must_be_finite_positive(lib):
    for s in (float("nan"), float("inf"), 0.0, -0.5):
        assert fwd(lib, scale=s) == fa.FA_ERR_INVALID_ARG
        assert dkdv(lib, scale=s) == fa.FA_ERR_INVALID_ARG
        assert dq(lib, scale=s) == fa.FA_ERR_INVALID_ARG


def test_tilings(lib):
    # bf16: only the tuned tilings
    assert fwd(lib, bm=64, bn=64, q=0) == fa.FA_ERR_UNSUPPORTED    # tiling is checked before pointers
    assert dkdv(lib, bm=256, bn=128, q=0) == fa.FA_ERR_UNSUPPORTED
    assert dkdv(lib, bm=128, bn=128, q=0) == fa.FA_ERR_INVALID_ARG   # d = 64 has it; then null q
    assert dq(lib, bm=16, bn=16, q=0) == fa.FA_ERR_UNSUPPORTED
    assert fwd(lib, bm=-1, bn=0) == fa.FA_ERR_INVALID_ARG
    # float32: block_m in {16,32,64,128}, block_n multiple of 4 up to 128, LDS budget
    f32 = dict(dtype=fa.FA_F32, d=16, q=0)
    assert fwd(lib, bm=16, bn=12, **f32) == fa.FA_ERR_INVALID_ARG           # accepted tiling, then null q
    assert fwd(lib, bm=48, bn=16, **f32) == fa.FA_ERR_UNSUPPORTED
    assert fwd(lib, bm=16, bn=14, **f32) == fa.FA_ERR_UNSUPPORTED
    assert fwd(lib, bm=16, bn=132, **f32) == fa.FA_ERR_UNSUPPORTED
    assert dkdv(lib, bm=128, bn=128, dtype=fa.FA_F32, d=128, q=0) == fa.FA_ERR_INVALID_ARG  # 129 KiB fits
    for bm, bn in ((16, 12), (16, 16), (32, 64), (64, 32), (128, 128)):
        assert dq(lib, bm=bm, bn=bn, dtype=fa.FA_F32, d=32, q=0) == fa.FA_ERR_INVALID_ARG


def rect(lib, fn, **kw):
    a = dict(q=A, k=B, v=C, dO=D_, lse=E, delta=F, o=D_, dq=G, dk=G, dv=H, bh=1, nq=64, nk=128, d=64,
             dtype=fa.FA_BF16, scale=0.125, causal=1, window=0, bm=0, bn=0)
    a.update(kw)
    if fn == "fwd":
        return lib.fa_fwd_rect(a["q"], a["k"], a["v"], a["o"], a["lse"], a["bh"], a["nq"], a["nk"], a["d"],
                               a["dtype"], a["scale"], a["causal"], a["window"], a["bm"], a["bn"], None)
    if fn == "dkdv":
        return lib.fa_bwd_dkdv_rect(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dk"], a["dv"],
                                    a["bh"], a["nq"], a["nk"], a["d"], a["dtype"], a["scale"], a["causal"],
                                    a["window"], a["bm"], a["bn"], None)
    return lib.fa_bwd_dq_rect(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dq"], a["bh"],
                              a["nq"], a["nk"], a["d"], a["dtype"], a["scale"], a["causal"], a["window"],
                              a["bm"], a["bn"], None)


def test_rect_lengths(lib):
    for fn in ("fwd", "dkdv", "dq"):
        # causal needs every query to see a key: nq <= nk
        assert rect(lib, fn, nq=129, nk=128) == fa.FA_ERR_UNSUPPORTED
        assert rect(lib, fn, nq=129, nk=128, causal=0, q=0) == fa.FA_ERR_INVALID_ARG   # accepted, then null q
        # exactly one empty length has no meaning; both empty (or bh = 0) is a no-op
        assert rect(lib, fn, nq=0, nk=5) == fa.FA_ERR_INVALID_ARG
        assert rect(lib, fn, nq=5, nk=0, causal=0) == fa.FA_ERR_INVALID_ARG
        assert rect(lib, fn, nq=0, nk=0, q=0, k=0) == fa.FA_OK
        assert rect(lib, fn, bh=0, q=0, k=0) == fa.FA_OK
        assert rect(lib, fn, nq=-1) == fa.FA_ERR_INVALID_ARG
        assert rect(lib, fn, nk=(1 << 24) + 1, causal=0) == fa.FA_ERR_UNSUPPORTED
        assert rect(lib, fn, q=A + 2) == fa.FA_ERR_MISALIGNED


def test_rect_window_arguments(lib):
    for fn in ("fwd", "dkdv", "dq"):
        # a window is a positive key count, and only narrows causal attention
        assert rect(lib, fn, window=-1) == fa.FA_ERR_INVALID_ARG
        assert rect(lib, fn, window=16, causal=0) == fa.FA_ERR_INVALID_ARG
        assert rect(lib, fn, window=-1, bh=0, q=0, k=0) == fa.FA_ERR_INVALID_ARG
        # valid windows (any size, including wider than the keys) pass the
        # argument checks and stop at the null q
        for window in (1, 100, 128, 1 << 30, (1 << 31) - 1):
            assert rect(lib, fn, window=window, q=0) == fa.FA_ERR_INVALID_ARG
            assert rect(lib, fn, window=window, bh=0, q=0, k=0) == fa.FA_OK


def test_empty_input_is_noop(lib):
    # bh == 0 or n == 0: nothing to do, pointers are not touched
    assert fwd(lib, q=0, k=0, v=0, o=0, lse=0, bh=0) == fa.FA_OK
    assert fwd(lib, q=0, k=0, v=0, o=0, lse=0, n=0) == fa.FA_OK
    assert dkdv(lib, q=0, dk=0, n=0) == fa.FA_OK
    assert dq(lib, q=0, dq=0, bh=0) == fa.FA_OK
    assert lib.fa_bwd_preprocess(0, 0, 0, 0, 64, 64, fa.FA_BF16, None) == fa.FA_OK


def test_outputs_must_not_alias(lib):
    assert fwd(lib, o=A) == fa.FA_ERR_INVALID_ARG
    assert fwd(lib, lse=D_) == fa.FA_ERR_INVALID_ARG
    assert dkdv(lib, dk=H) == fa.FA_ERR_INVALID_ARG
    assert dkdv(lib, dv=B) == fa.FA_ERR_INVALID_ARG
    assert dq(lib, dq=F) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_preprocess(A, B, A, 1, 64, 64, fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, causal=True)


def test_autograd_op_validates_on_host():
    import torch
    q = torch.zeros(2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.flash_attention(q, q, q)                      # host tensors are refused
    with pytest.raises(ValueError):
        fa.flash_attention(q, q[:, :, :32], q[:, :, :32])  # head dims must agree
    with pytest.raises(ValueError):
        fa.flash_attention(q, q[:1], q[:1])              # leading dims must agree
    with pytest.raises(ValueError):
        fa.flash_attention(q[0, 0], q[0, 0], q[0, 0])    # needs [..., n, d]


# --------------------------------------------------------------------------- fused backward
W = 0x90000   # fake workspace address


def fused(lib, **kw):
    a = dict(q=A, k=B, v=C, dO=D_, lse=E, delta=F, dq=G, dk=H, dv=0xA0000, ws=W, bh=1, nq=64, nk=128, d=64,
             dtype=fa.FA_BF16, scale=0.125, causal=1, window=0, bm=0, bn=0)
    a.update(kw)
    return lib.fa_bwd_fused(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dq"], a["dk"], a["dv"],
                            a["ws"], a["bh"], a["nq"], a["nk"], a["d"], a["dtype"], a["scale"], a["causal"],
                            a["window"], a["bm"], a["bn"], None)


def test_fused_workspace_bytes(lib):
    assert fa.fa_bwd_fused_workspace_bytes(32, 8192, 128, fa.FA_BF16) == 32 * 8192 * 128 * 4
    assert fa.fa_bwd_fused_workspace_bytes(32, 8192, 128, fa.FA_F32) == 0
    assert fa.fa_bwd_fused_workspace_bytes(0, 8192, 128, fa.FA_BF16) == 0
    assert fa.fa_bwd_fused_workspace_bytes(-1, 8192, 128, fa.FA_BF16) == 0
    # no 32-bit overflow at the largest sizes
    assert fa.fa_bwd_fused_workspace_bytes(1 << 20, 1 << 24, 128, fa.FA_BF16) == (1 << 20) * (1 << 24) * 512


def test_fused_tiles(lib):
    assert fa.fa_default_tiles(fa.FA_BF16, 128, fa.KERNEL_FUSED) == (64, 128)
    assert fa.fa_default_tiles(fa.FA_BF16, 64, fa.KERNEL_FUSED) == (64, 128)
    assert fa.fa_default_tiles(fa.FA_F32, 32, fa.KERNEL_FUSED) == (64, 64)
    # the 128-query bf16 dK/dV tiling does not leave LDS for the fused dQ operands
    assert fused(lib, d=128, bm=128, bn=128) == fa.FA_ERR_UNSUPPORTED
    assert fused(lib, dtype=fa.FA_F32, d=128, bm=48, bn=64) == fa.FA_ERR_UNSUPPORTED


def test_fused_argument_checks(lib):
    assert fused(lib, ws=0) == fa.FA_ERR_INVALID_ARG                 # bf16 needs the workspace
    assert fused(lib, ws=W + 4) == fa.FA_ERR_MISALIGNED
    assert fused(lib, ws=G) == fa.FA_ERR_INVALID_ARG                 # workspace is dq
    assert fused(lib, ws=A) == fa.FA_ERR_INVALID_ARG                 # workspace is q
    assert fused(lib, dq=A) == fa.FA_ERR_INVALID_ARG
    assert fused(lib, dq=H) == fa.FA_ERR_INVALID_ARG                 # dq is dk
    assert fused(lib, dq=0) == fa.FA_ERR_INVALID_ARG
    assert fused(lib, window=-1) == fa.FA_ERR_INVALID_ARG
    assert fused(lib, window=5, causal=0) == fa.FA_ERR_INVALID_ARG
    assert fused(lib, nq=129, nk=128) == fa.FA_ERR_UNSUPPORTED
    assert fused(lib, scale=0.0) == fa.FA_ERR_INVALID_ARG
    assert fused(lib, bh=0, q=0, ws=0) == fa.FA_OK
    assert fused(lib, d=96) == fa.FA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------- plain C client
def test_c_client_links_and_reports_abi(lib):
    """The C99 client of include/fa.h (built by build()) links against
    libfa.so and calls its host-only functions without Python in between."""
    import subprocess
    from exact_tiled_attention_26_amd.build import C_CLIENT
    assert os.path.exists(C_CLIENT), "build the C client first (__graft_entry__.build())"
    r = subprocess.run([C_CLIENT, "--abi"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[:2] == ["abi", str(fa.fa_abi_version())]
    # bad arguments are refused before any HIP call
    r = subprocess.run([C_CLIENT, "in", "out", "0", "8", "64", "1"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1


def noalloc(lib, **kw):
    a = dict(q=A, k=B, v=C, dO=D_, lse=E, delta=F, dq=G, dk=H, dv=0x90000, bh=1, nq=64, nk=64, d=64,
             dtype=fa.FA_BF16, scale=0.125, causal=1, window=0, bm=0, bn=0)
    a.update(kw)
    return lib.fa_bwd_fused_noalloc(a["q"], a["k"], a["v"], a["dO"], a["lse"], a["delta"], a["dq"], a["dk"],
                                    a["dv"], a["bh"], a["nq"], a["nk"], a["d"], a["dtype"], a["scale"],
                                    a["causal"], a["window"], a["bm"], a["bn"], None)


def test_noalloc_rejects_what_exceeds_its_scratch(lib):
    """The allocation-free backward's fixed scratch holds bh * nq * d float32
    values up to FA_NOALLOC_SCRATCH_BYTES; a larger bf16 call is refused on
    the host, before any HIP call (the fake pointers are never touched)."""
    cap = fa.FA_NOALLOC_SCRATCH_BYTES // 4
    assert noalloc(lib, bh=cap // (8192 * 128) + 1, nq=8192, nk=8192, d=128) == fa.FA_ERR_TOO_LARGE
    assert noalloc(lib, bh=1, nq=cap // 64 + 1, nk=cap // 64 + 1, d=64) == fa.FA_ERR_TOO_LARGE
    assert "scratch" in fa.fa_status_str(fa.FA_ERR_TOO_LARGE)
    # the usual argument checks come first and are those of fa_bwd_fused
    assert noalloc(lib, dq=0) == fa.FA_ERR_INVALID_ARG
    assert noalloc(lib, dq=A) == fa.FA_ERR_INVALID_ARG
    assert noalloc(lib, dk=0x90008) == fa.FA_ERR_MISALIGNED
    assert noalloc(lib, d=96) == fa.FA_ERR_UNSUPPORTED
    assert noalloc(lib, bm=64, bn=64) == fa.FA_ERR_UNSUPPORTED
    assert noalloc(lib, window=8, causal=0) == fa.FA_ERR_INVALID_ARG
    assert noalloc(lib, bh=0) == fa.FA_OK
