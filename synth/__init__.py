"""Seeded synthetic inputs for the parallel-draft step.

This package only *generates data*: model shapes, random weights, a verified
batch, a paged KV cache and the uniform draws used to build target tokens.  It
holds none of the drafting method's arithmetic (no expansion, no forward pass,
no acceptance), so that the CPU oracle and the HIP path can both consume the
same inputs without sharing any computation.
"""

from .workloads import (  # noqa: F401
    ModelSpec,
    TINY,
    GPTOSS20B,
    QWEN3CODER30B,
    Workload,
    WORKLOADS,
    Batch,
    make_weights,
    make_batch,
    make_agreement_draws,
    target_tokens_from_drafts,
    store,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    NAN_BF16_BITS,
)
