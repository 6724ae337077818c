"""P-EAGLE parallel-draft step on AMD MI355X (gfx950).

Public API (thin ctypes binding over libpeagle.so; all work runs in HIP):

* :class:`DraftModel` -- drafter shape + borrowed device weights
* :func:`prepare_draft_batch` -- expand the verified batch, place hidden states
* :func:`draft_forward` -- one drafter pass producing K tokens per sequence
* :func:`draft_forward_noalloc` -- the same pass on the library's static scratch (no workspace)
* :func:`accept` -- greedy accepted length and next bonus token
* :func:`draft_autoregressive` -- the K-pass autoregressive baseline on the same kernels
* :func:`next_verified_batch` -- next round's verified batch from this round's results
* :func:`check_verified_batch` -- device check of a verified batch's preconditions
"""

from ._lib import (  # noqa: F401
    DraftModel,
    PeError,
    accept,
    check_verified_batch,
    draft_autoregressive,
    draft_forward,
    draft_forward_noalloc,
    load,
    next_verified_batch,
    prepare_draft_batch,
    status_string,
    timing_enable,
    timing_read,
    PE_KERNEL_LM_HEAD,
    PE_KERNEL_PREPARE,
    PE_KERNEL_ATTENTION,
    PE_CHECK_QUERY_LEN,
    PE_CHECK_ACCEPTED,
    PE_CHECK_TOKEN_ID,
    PE_CHECK_POSITION,
    PE_CHECK_BLOCK_TABLE,
)
