"""fp64 CPU oracle for fused linear cross-entropy (FLCE).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``linear_cross_entropy_gemm_amd``) never imports it
and shares no code with it; the only module both sides use is ``synth``, which
draws the seeded inputs and holds none of the method's arithmetic.

The oracle is the plain definition of what FLCE computes (FLCE reaches the same
result as the unfused projection + cross-entropy, only without materialising
the logits), written out in float64 with no blocking beyond splitting rows into
independent blocks.  Every function is pinned by ``tests/test_oracle.py``
against closed forms, invariants, a library routine on special cases, brute
force and central finite differences.

Parity unpinned: none of the functions here is unpinned.  At full lm_head sizes
the GPU path is checked on sampled rows (``grad_h``) and sampled vocabulary rows
(``grad_W``); entries outside the samples are covered only by the column-sum
invariant on configs without a softcap.
"""
from .flce import (  # noqa: F401
    capped_logits,
    cross_entropy_on_logits,
    flce_reference,
    row_stats,
    grad_h_rows,
    grad_W_rows,
    n_correct_window,
    reduction_scale,
)
