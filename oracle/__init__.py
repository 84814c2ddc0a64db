"""Plain, slow CPU oracle for the multi-head attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports,
calls or links it, and this package imports nothing from the product path.

Modules
-------
mha_oracle   dense float64 reference: projections (two independent forms),
             materialised score matrix, mask, stable row softmax, weighted
             value sum, head concatenation, output projection; and the
             analytic gradients of the attention core.
summary      the stable key-block summary (m, l, z), its empty state and its
             merge rule, written out literally for checking identities.
bruteforce   pure-Python scalar loops in 50-digit mpmath arithmetic for tiny
             shapes; shares no code with ``mha_oracle``.

Every function is pinned by the CPU tests in ``tests/test_oracle_pins.py``
against values the pages print, closed forms, invariants and the brute force.
"""

from .mha_oracle import (  # noqa: F401
    EmptyRowError,
    allowed_set,
    project_separate,
    project_combined,
    masked_softmax_rows,
    attn_core_ref,
    attn_core_grad_ref,
    mha_ref,
    mha_ref_rows,
    mha_grad_ref,
)
from .summary import BOTTOM, summary, merge, finalize, fold  # noqa: F401
