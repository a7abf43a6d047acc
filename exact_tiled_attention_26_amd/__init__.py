"""Exact tiled (Flash) attention for one MI355X (gfx950): forward and backward.

The computation lives in ``libfa.so`` (hand-written HIP kernels behind the C
ABI of ``include/fa.h``); this package is its thin ctypes binding.  PyTorch
is used only for device memory and streams.
"""

from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARG,
    FA_ERR_MISALIGNED,
    FA_ERR_TOO_LARGE,
    FA_ERR_UNSUPPORTED,
    FA_NOALLOC_SCRATCH_BYTES,
    FA_OK,
    KERNEL_DKDV,
    KERNEL_DQ,
    KERNEL_FUSED,
    KERNEL_FWD,
    LIB_PATH,
    SIGNATURES,
    FAError,
    backward,
    backward_fused,
    fa_abi_version,
    fa_bwd_fused,
    fa_bwd_fused_noalloc,
    fa_bwd_fused_workspace_bytes,
    fa_bwd_dkdv,
    fa_bwd_dq,
    fa_bwd_dq_rect,
    fa_bwd_dkdv_rect,
    fa_bwd_preprocess,
    fa_default_tiles,
    fa_fwd,
    fa_fwd_rect,
    fa_status_str,
    forward,
    load_library,
)
from .autograd import FlashAttention, flash_attention  # noqa: F401
