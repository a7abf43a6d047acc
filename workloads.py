"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle.

This module holds no attention arithmetic: it only draws random numbers,
casts them to the I/O dtype and upcasts them back.  Both the GPU path and the
CPU oracle read the *cast* tensors, so input rounding is never charged to the
kernel.

Recipe (every workload): ``numpy.random.default_rng(seed)`` (seed 0 unless
stated), then four fp64 ``standard_normal`` draws in the order Q, K, V, dO,
each of shape [BH, N, d], then a cast to fp32 or bf16 (round to nearest even)
by torch.  For the single-head gradient-check workload this reproduces the
draws of the gradient check in "CS349E lecture 11, 03_flash_backward.py"
(demo1_gradcheck: default_rng(0), Q, K, V then G, each 48 x 16).

The pages measure on no public dataset; these synthetic N(0, 1) tensors are
the workloads, at the shapes the pages and the target configuration name.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    bh: int
    n: int
    d: int
    dtype: str                      # "fp32" | "bf16"
    causal: tuple = (False, True)
    tiles: tuple = ()               # (block_m, block_n) pairs; () = library default
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "gradcheck_48": Workload(
        "gradcheck_48", 1, 48, 16, "fp32", (False, True), ((16, 12),),
        "single head, tiles 16 x 12, fwd+bwd, oracle + finite differences"),
    "tile_sweep_256": Workload(
        "tile_sweep_256", 4, 256, 32, "fp32", (False, True),
        ((16, 16), (32, 64), (64, 32), (128, 128)),
        "output must not depend on the tile size"),
    "bf16_2048_d64": Workload(
        "bf16_2048_d64", 32, 2048, 64, "bf16", (True,), (),
        "batch 4 x 8 heads, fp32 accumulation"),
    "headline_8192_d128": Workload(
        "headline_8192_d128", 32, 8192, 128, "bf16", (True, False), (),
        "batch*heads 32, the throughput workload"),
    "long_32768_d128": Workload(
        "long_32768_d128", 8, 32768, 128, "bf16", (True,), (),
        "long context; only L is saved, never P"),
    # throughput of the float32 kernels (not one of the pages' configurations)
    "fp32_4096_d64": Workload(
        "fp32_4096_d64", 16, 4096, 64, "fp32", (True, False), (),
        "float32 I/O and products, for the float32 kernels' throughput"),
}


def make_inputs(bh: int, n: int, d: int, seed: int = 0):
    """Return fp64 arrays (q, k, v, do), each [bh, n, d], drawn in that order."""
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((bh, n, d)) for _ in range(4))


def make_rect_inputs(bh: int, nq: int, nk: int, d: int, seed: int = 0):
    """Like make_inputs for nq queries against nk keys: fp64 arrays drawn in
    the order q [bh, nq, d], k [bh, nk, d], v [bh, nk, d], do [bh, nq, d]."""
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((bh, rows, d)) for rows in (nq, nk, nk, nq))


def torch_dtype(name: str):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def cast_io(arrays, dtype: str, device="cpu"):
    """Cast fp64 numpy arrays to torch tensors of the I/O dtype (contiguous)."""
    import torch
    td = torch_dtype(dtype)
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(td).to(device).contiguous()
                 for a in arrays)


def to_f64(t) -> np.ndarray:
    """Exact fp64 copy of a torch tensor (any device, fp32 or bf16)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
