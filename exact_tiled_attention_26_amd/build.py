"""Build libfa.so (the C-ABI library of HIP kernels for gfx950) in place.

Usage: ``python -m exact_tiled_attention_26_amd.build`` or ``build()`` from
Python.  Every source under ``csrc/`` is compiled with hipcc for gfx950 into
``_build/`` (in parallel) and linked into ``libfa.so`` next to this file.
``build_c_client()`` also compiles the plain C client of the ABI that the
tests run (``tests/c_abi/fa_c_client.c``, host code only, linked against
libfa.so), and ``build_order_check()`` the host-side check of the workgroup
order (``tests/c_abi/order_check.cpp``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libfa.so")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


ROOT = os.path.dirname(HERE)
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "fa_c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_abi", "_build", "fa_c_client")


def build_c_client(verbose: bool = False) -> str:
    """Compile the C99 client of include/fa.h with the host C compiler; it
    finds libfa.so next to this file through a relative run path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc) for the C client of the ABI")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(os.path.dirname(C_CLIENT), exist_ok=True)
    rpath = "$ORIGIN/" + os.path.relpath(HERE, os.path.dirname(C_CLIENT))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{os.path.join(ROOT, 'include')}", C_CLIENT_SRC, f"-L{HERE}", "-lfa", f"-L{rocm}/lib",
           "-lamdhip64", f"-Wl,-rpath,{rpath}:{rocm}/lib", "-lm", "-o", C_CLIENT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CLIENT}")
    return C_CLIENT


ORDER_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "order_check.cpp")
ORDER_CHECK = os.path.join(ROOT, "tests", "c_abi", "_build", "order_check")


def build_order_check(verbose: bool = False) -> str:
    """Compile the host-side check of the workgroup order (csrc/fa_order.h)
    with hipcc as host code only; it runs on the CPU."""
    os.makedirs(os.path.dirname(ORDER_CHECK), exist_ok=True)
    cmd = [_hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "--offload-host-only", "-O2", "-std=c++17",
           "-Wall", ORDER_CHECK_SRC, "-o", ORDER_CHECK]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"order check build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {ORDER_CHECK}")
    return ORDER_CHECK


SWIZZLE_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "swizzle_check.cpp")
SWIZZLE_CHECK = os.path.join(ROOT, "tests", "c_abi", "_build", "swizzle_check")


def build_swizzle_check(verbose: bool = False) -> str:
    """Compile the host-side check of the bf16 LDS tile layout (the copy
    placement, the readers' offsets and the bank model in csrc/fa_common.h)
    with hipcc as host code only; it runs on the CPU."""
    os.makedirs(os.path.dirname(SWIZZLE_CHECK), exist_ok=True)
    cmd = [_hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "--offload-host-only", "-O2", "-std=c++17",
           "-Wall", SWIZZLE_CHECK_SRC, "-o", SWIZZLE_CHECK]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"swizzle check build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SWIZZLE_CHECK}")
    return SWIZZLE_CHECK


if __name__ == "__main__":
    build(verbose=True)
    build_c_client(verbose=True)
    build_order_check(verbose=True)
    build_swizzle_check(verbose=True)
    sys.exit(0)
