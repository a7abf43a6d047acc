"""Host-side check of the bf16 LDS tile layout
(exact_tiled_attention_26_amd/csrc/fa_common.h): tests/c_abi/swizzle_check.cpp,
compiled by __graft_entry__.build() as host code only, checks on the CPU that
the asynchronous tile copy places every 16-byte chunk exactly once, that the
natural and transposed operand readers find each element where the copy put
it (the transposed read in the row order ds_read_b64_tr_b16 transposes), and
that under the bank model stated in fa_common.h (64 banks of 4 bytes; 16
lanes per clock for ds_read_b128, 32 for ds_read_b64_tr_b16) neither read
has a bank conflict, for every tile height and row origin the bf16 kernels
use at head dims 64 and 128.  The counters of the same kernels on the device
(SQ_LDS_BANK_CONFLICT, profiles/) read zero."""

import os
import subprocess

from exact_tiled_attention_26_amd.build import SWIZZLE_CHECK, build_swizzle_check


def test_lds_tile_layout_host_check():
    exe = SWIZZLE_CHECK if os.path.exists(SWIZZLE_CHECK) else build_swizzle_check()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("swizzle ok:"), r.stdout
    assert int(r.stdout.split()[2]) > 10000
