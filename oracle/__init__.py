"""CPU oracle for In-context Sparse Attention (ISA) -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain fp64 reference that the HIP path is checked
against.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  The product path (the C-ABI library and its Python
binding) never imports, calls or links anything here, and the oracle shares no
code, tables or helpers with the HIP kernels.

Modules:
  isa_oracle  vectorised fp64 NumPy implementation of every step
  brute       pure-Python loop implementation for tiny inputs (a second,
              independent writing of the same definitions)

Which parts are pinned, and by what, is listed in the header of
``isa_oracle``.  The one part with no external pin is flagged there as
"parity unpinned".
"""

from .isa_oracle import (  # noqa: F401
    count_rule,
    block_ranges,
    pool_blocks,
    saliency_scores,
    top_indices,
    sharpness_scores,
    full_attention_rows,
    taylor_attention_rows,
    dense_attention,
    oracle_plan_head,
    oracle_forward_head,
    oracle_plan,
    oracle_forward,
    isa_reference,
)
