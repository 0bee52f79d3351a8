"""fp64 CPU oracle for causal and packed-document scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time against the
HIP kernels.  It shares no code with the kernels, their headers or their
Python binding.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` (closed forms, invariants, finite differences, a
library cross-check); none is "parity unpinned".
"""
from .attention import (  # noqa: F401
    MASK_CAUSAL,
    MASK_DOC_CAUSAL,
    allowed_mask,
    attention_fwd_ref,
    attention_bwd_ref,
    attention_decode_ref,
    attention_fwd_rows_ref,
    attention_dq_rows_ref,
    attention_dkdv_rows_ref,
    delta_ref,
)
from .rope import (  # noqa: F401
    ROPE_BASE,
    attention_rope_ref,
    rope_angles,
    rope_positions,
    rope_rotate,
    round_to_dtype,
)
