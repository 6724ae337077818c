"""CPU oracle for the P-EAGLE parallel-draft step (test infrastructure).

Plain, slow, float64 numpy definitions of what one parallel-draft round
computes.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path never does.  It shares no
code with the HIP library and does not import it.

Every function is pinned by CPU tests against facts fixed by the method's
description and by mathematics (invariants, closed forms, brute force,
independent library compositions); see ``tests/test_oracle_*.py``.
"""

from .peagle_oracle import (  # noqa: F401
    PADDING_SLOT_ID,
    decode,
    encode,
    round_operand,
    expand_batch,
    scatter_broadcast,
    rms_norm,
    rope_rotate_half,
    silu,
    paged_attention,
    draft_forward,
    accept,
    parallel_draft_step,
    apply_cache_writes,
    next_verified_batch,
    autoregressive_draft,
)
