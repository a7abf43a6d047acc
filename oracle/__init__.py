"""CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously correct fp64 reference that the GPU path
is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library
(``exact_tiled_attention_26_amd``) never imports it, and it imports nothing
from the product: the two share no code.  The only module both sides use is
``workloads`` (seeded synthetic inputs, no attention arithmetic).

Sources, cited by page title and section throughout:

* [CS336-A2] "Assignment2: FlashAttention & Distributed Data Parallel notes",
  Part 1 (section 1.1 standard attention, 1.2 FA-2 forward, 1.3 Triton
  forward with causal tile skipping, 1.4 backward Eq 13-19 and the
  two-kernel backward).
* [CS349E-L11] "CS349E lecture 11, 03_flash_backward.py" (demo1_gradcheck,
  demo2_memory, demo3_fwd_bwd_cost, demo4_causal).
* [CS324-L8] "CS324 lecture 8, 03_online_softmax_and_flash.py"
  (demo1_overflow, demo2_online, demo3_forward, demo4_backward,
  flash_attention_torch, window_attention_torch).

Modules:

* ``oracle.attention`` -- the direct definition (materialises S and P per
  head, in row chunks).  This is what the GPU is compared with.
* ``oracle.tiled``     -- an fp64 CPU model of the tiled algorithm (online
  softmax, Br x Bc tiles, causal tile skipping, two-loop backward) with a
  tile counter.  It is used only to check the pages' claims against
  ``oracle.attention``; it is never a GPU reference.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
things other than itself: central finite differences, torch CPU fp64
autograd and ``scaled_dot_product_attention``, ``scipy.special.logsumexp``,
the online-softmax worked example, closed-form special cases, invariants and
the causal tile-count formula.  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    delta_from_output,
    forward_rows,
    dq_rows,
    dkdv_cols,
    head_row_stats,
)
from .tiled import (  # noqa: F401
    online_softmax,
    tiled_forward,
    tiled_backward,
    causal_tiles_computed,
)
