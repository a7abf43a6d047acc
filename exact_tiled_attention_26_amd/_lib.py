"""ctypes binding of libfa.so: the entry points of include/fa.h, by the same names.

Argument marshalling only.  Every function takes torch tensors (device
memory) and passes their data pointers, sizes and the current HIP stream to
the C ABI; every step of the computation runs in the library's kernels.
There is no fallback: if libfa.so is missing or fails to load, every call
raises.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F32, FA_BF16 = 0, 1
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_MISALIGNED, FA_ERR_HIP, FA_ERR_TOO_LARGE = range(6)
FA_NOALLOC_SCRATCH_BYTES = 1 << 27   # FA_NOALLOC_SCRATCH_BYTES of include/fa.h
KERNEL_FWD, KERNEL_DKDV, KERNEL_DQ, KERNEL_FUSED = 0, 1, 2, 3

# (name, argtypes) for every function include/fa.h declares
_P, _I, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "fa_fwd": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P],
    "fa_bwd_preprocess": [_P, _P, _P, _I, _I, _I, _I, _P],
    "fa_bwd_dkdv": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P],
    "fa_bwd_dq": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P],
    "fa_fwd_rect": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P],
    "fa_bwd_dkdv_rect": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P],
    "fa_bwd_dq_rect": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P],
    "fa_bwd_fused": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P],
    "fa_bwd_fused_workspace_bytes": [_I, _I, _I, _I],
    "fa_bwd_fused_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P],
    "fa_default_tiles": [_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)],
    "fa_status_str": [_I],
    "fa_abi_version": [],
}


class FAError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func} failed: status {status} ({msg})")
        self.status = status


_lib = None
ABI_VERSION = 5   # FA_ABI_VERSION of include/fa.h that SIGNATURES describe


def load_library(path: str = LIB_PATH):
    """Load libfa.so once; raises if it is missing (build it with
    ``python -m exact_tiled_attention_26_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build the HIP library first "
                           "(python -m exact_tiled_attention_26_amd.build)")
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"fa_status_str": ctypes.c_char_p,
                      "fa_bwd_fused_workspace_bytes": ctypes.c_size_t}.get(name, ctypes.c_int)
    if lib.fa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI {lib.fa_abi_version()}, the binding expects {ABI_VERSION}: "
                           "rebuild the HIP library")
    _lib = lib
    return lib


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def fa_default_tiles(dtype: int, d: int, kernel: int):
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    st = load_library().fa_default_tiles(int(dtype), int(d), int(kernel), ctypes.byref(bm), ctypes.byref(bn))
    _check("fa_default_tiles", st)
    return bm.value, bn.value


def _check(func: str, status: int):
    if status != FA_OK:
        raise FAError(func, status, fa_status_str(status))


# ------------------------------------------------------------------ tensor marshalling
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _shape3(q):
    if q.dim() != 3:
        raise ValueError(f"expected a [bh, n, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_io(ref, tensors, name_dtype, kref=None):
    """Device, contiguity, dtype and shape checks: "io" tensors match ref (q),
    "kv" tensors match kref (k; default ref) in shape and ref in dtype, "row"
    tensors are float32 [bh, n] with ref's bh and n."""
    import torch
    kref = ref if kref is None else kref
    for name, t, want in tensors:
        _require(t.is_cuda, f"{name} must be a device tensor")
        _require(t.is_contiguous(), f"{name} must be contiguous")
        if want in ("io", "kv"):
            shape = ref.shape if want == "io" else kref.shape
            _require(t.dtype == ref.dtype and tuple(t.shape) == tuple(shape),
                     f"{name} must match {'q' if want == 'io' else 'k'} in shape and q in dtype")
        else:
            _require(t.dtype == torch.float32 and tuple(t.shape) == tuple(ref.shape[:2]),
                     f"{name} must be float32 of shape [bh, n]")


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def fa_fwd(q, k, v, o, lse, causal: bool, scale: float | None = None,
           block_m: int = 0, block_n: int = 0, stream=None):
    """Forward: writes o and lse in place (see include/fa.h)."""
    bh, n, d = _shape3(q)
    _check_io(q, [("q", q, "io"), ("k", k, "io"), ("v", v, "io"), ("o", o, "io"), ("lse", lse, "row")], None)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), bh, n, d, _dtype_code(q),
                               scale, int(bool(causal)), int(block_m), int(block_n), _stream(stream))
    _check("fa_fwd", st)


def fa_bwd_preprocess(o, dO, delta, stream=None):
    """D = rowsum(O * dO): writes delta in place."""
    bh, n, d = _shape3(o)
    _check_io(o, [("o", o, "io"), ("dO", dO, "io"), ("delta", delta, "row")], None)
    st = load_library().fa_bwd_preprocess(_ptr(o), _ptr(dO), _ptr(delta), bh, n, d, _dtype_code(o),
                                          _stream(stream))
    _check("fa_bwd_preprocess", st)


def fa_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, causal: bool, scale: float | None = None,
                block_m: int = 0, block_n: int = 0, stream=None):
    """dK, dV (key/value-tile outer kernel): writes dk and dv in place."""
    bh, n, d = _shape3(q)
    _check_io(q, [("q", q, "io"), ("k", k, "io"), ("v", v, "io"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dk", dk, "io"), ("dv", dv, "io")], None)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dk),
                                    _ptr(dv), bh, n, d, _dtype_code(q), scale, int(bool(causal)),
                                    int(block_m), int(block_n), _stream(stream))
    _check("fa_bwd_dkdv", st)


def fa_bwd_dq(q, k, v, dO, lse, delta, dq, causal: bool, scale: float | None = None,
              block_m: int = 0, block_n: int = 0, stream=None):
    """dQ (query-tile outer kernel): writes dq in place."""
    bh, n, d = _shape3(q)
    _check_io(q, [("q", q, "io"), ("k", k, "io"), ("v", v, "io"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dq", dq, "io")], None)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dq),
                                  bh, n, d, _dtype_code(q), scale, int(bool(causal)), int(block_m),
                                  int(block_n), _stream(stream))
    _check("fa_bwd_dq", st)


def _kv_shape(q, k):
    bh, _, d = _shape3(q)
    bhk, nk, dk = _shape3(k)
    _require(bhk == bh and dk == d, "k must be [bh, nk, d] with q's bh and d")
    return nk


def fa_fwd_rect(q, k, v, o, lse, causal: bool, scale: float | None = None,
                block_m: int = 0, block_n: int = 0, stream=None, window: int = 0):
    """Forward for q [bh, nq, d] against k, v [bh, nk, d]; causal masking is
    aligned to the end of the keys, and ``window`` > 0 (causal only) keeps
    each query's ``window`` most recent keys (see include/fa.h)."""
    bh, nq, d = _shape3(q)
    nk = _kv_shape(q, k)
    _check_io(q, [("q", q, "io"), ("k", k, "kv"), ("v", v, "kv"), ("o", o, "io"), ("lse", lse, "row")],
              None, kref=k)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), bh, nq, nk, d,
                                    _dtype_code(q), scale, int(bool(causal)), int(window), int(block_m),
                                    int(block_n), _stream(stream))
    _check("fa_fwd_rect", st)


def fa_bwd_dkdv_rect(q, k, v, dO, lse, delta, dk, dv, causal: bool, scale: float | None = None,
                     block_m: int = 0, block_n: int = 0, stream=None, window: int = 0):
    """dK, dV for q, dO [bh, nq, d] against k, v [bh, nk, d]."""
    bh, nq, d = _shape3(q)
    nk = _kv_shape(q, k)
    _check_io(q, [("q", q, "io"), ("k", k, "kv"), ("v", v, "kv"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dk", dk, "kv"), ("dv", dv, "kv")], None, kref=k)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dkdv_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta),
                                         _ptr(dk), _ptr(dv), bh, nq, nk, d, _dtype_code(q), scale,
                                         int(bool(causal)), int(window), int(block_m), int(block_n),
                                         _stream(stream))
    _check("fa_bwd_dkdv_rect", st)


def fa_bwd_dq_rect(q, k, v, dO, lse, delta, dq, causal: bool, scale: float | None = None,
                   block_m: int = 0, block_n: int = 0, stream=None, window: int = 0):
    """dQ for q, dO [bh, nq, d] against k, v [bh, nk, d]."""
    bh, nq, d = _shape3(q)
    nk = _kv_shape(q, k)
    _check_io(q, [("q", q, "io"), ("k", k, "kv"), ("v", v, "kv"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dq", dq, "io")], None, kref=k)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dq_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta),
                                       _ptr(dq), bh, nq, nk, d, _dtype_code(q), scale, int(bool(causal)),
                                       int(window), int(block_m), int(block_n), _stream(stream))
    _check("fa_bwd_dq_rect", st)


def fa_bwd_fused_workspace_bytes(bh: int, nq: int, d: int, dtype: int) -> int:
    return int(load_library().fa_bwd_fused_workspace_bytes(int(bh), int(nq), int(d), int(dtype)))


def fa_bwd_fused(q, k, v, dO, lse, delta, dq, dk, dv, workspace, causal: bool, scale: float | None = None,
                 block_m: int = 0, block_n: int = 0, stream=None, window: int = 0):
    """Single-kernel backward: dK, dV and dQ (atomic adds) for q, dO
    [bh, nq, d] against k, v [bh, nk, d].  bf16 needs `workspace`, a float32
    device tensor of fa_bwd_fused_workspace_bytes bytes; float32 takes None."""
    import torch
    bh, nq, d = _shape3(q)
    nk = _kv_shape(q, k)
    _check_io(q, [("q", q, "io"), ("k", k, "kv"), ("v", v, "kv"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dq", dq, "io"), ("dk", dk, "kv"), ("dv", dv, "kv")], None, kref=k)
    if workspace is not None:
        _require(workspace.is_cuda and workspace.is_contiguous() and workspace.dtype == torch.float32,
                 "workspace must be a contiguous float32 device tensor")
        _require(workspace.numel() * 4 >= fa_bwd_fused_workspace_bytes(bh, nq, d, _dtype_code(q)),
                 "workspace is smaller than fa_bwd_fused_workspace_bytes")
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(workspace), bh, nq, nk, d, _dtype_code(q), scale,
                                     int(bool(causal)), int(window), int(block_m), int(block_n), _stream(stream))
    _check("fa_bwd_fused", st)


def fa_bwd_fused_noalloc(q, k, v, dO, lse, delta, dq, dk, dv, causal: bool, scale: float | None = None,
                         block_m: int = 0, block_n: int = 0, stream=None, window: int = 0):
    """fa_bwd_fused without a workspace: bf16 accumulates dQ in the library's
    fixed device scratch (FA_NOALLOC_SCRATCH_BYTES per GPU); calls that
    overlap on one GPU race on it."""
    bh, nq, d = _shape3(q)
    nk = _kv_shape(q, k)
    _check_io(q, [("q", q, "io"), ("k", k, "kv"), ("v", v, "kv"), ("dO", dO, "io"), ("lse", lse, "row"),
                  ("delta", delta, "row"), ("dq", dq, "io"), ("dk", dk, "kv"), ("dv", dv, "kv")], None, kref=k)
    scale = default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_fused_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dq),
                                             _ptr(dk), _ptr(dv), bh, nq, nk, d, _dtype_code(q), scale,
                                             int(bool(causal)), int(window), int(block_m), int(block_n),
                                             _stream(stream))
    _check("fa_bwd_fused_noalloc", st)


# ------------------------------------------------------------------ allocating helpers
def forward(q, k, v, causal: bool, scale=None, block_m=0, block_n=0, stream=None, window=0):
    """Allocate O and L with torch and run fa_fwd (fa_fwd_rect when k has a
    different length than q or a window is set); returns (o, lse)."""
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if tuple(k.shape) == tuple(q.shape) and not window:
        fa_fwd(q, k, v, o, lse, causal, scale, block_m, block_n, stream)
    else:
        fa_fwd_rect(q, k, v, o, lse, causal, scale, block_m, block_n, stream, window=window)
    return o, lse


def backward(q, k, v, o, dO, lse, causal: bool, scale=None, tiles_dkdv=(0, 0), tiles_dq=(0, 0),
             stream=None, window=0):
    """Allocate D, dQ, dK, dV with torch and run the three backward calls in
    order on one stream; returns (dq, dk, dv, delta)."""
    import torch
    delta = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_preprocess(o, dO, delta, stream)
    if tuple(k.shape) == tuple(q.shape) and not window:
        fa_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, causal, scale, *tiles_dkdv, stream=stream)
        fa_bwd_dq(q, k, v, dO, lse, delta, dq, causal, scale, *tiles_dq, stream=stream)
    else:
        fa_bwd_dkdv_rect(q, k, v, dO, lse, delta, dk, dv, causal, scale, *tiles_dkdv, stream=stream,
                         window=window)
        fa_bwd_dq_rect(q, k, v, dO, lse, delta, dq, causal, scale, *tiles_dq, stream=stream,
                       window=window)
    return dq, dk, dv, delta


def backward_fused(q, k, v, o, dO, lse, causal: bool, scale=None, tiles=(0, 0), stream=None, window=0):
    """Allocate D, dQ, dK, dV (and the bf16 workspace) with torch and run
    fa_bwd_preprocess then fa_bwd_fused on one stream; returns
    (dq, dk, dv, delta)."""
    import torch
    delta = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_bwd_fused_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], _dtype_code(q))
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device) if nbytes else None
    fa_bwd_preprocess(o, dO, delta, stream)
    fa_bwd_fused(q, k, v, dO, lse, delta, dq, dk, dv, ws, causal, scale, *tiles, stream=stream, window=window)
    return dq, dk, dv, delta
