"""Seeded synthetic inputs for draft-tree verification.

This module only draws inputs: trees (as parents arrays), candidate and
target tokens, prefix lengths and the q/k/v/cache tensors. It computes no
mask, no attention, no acceptance and no commit, so the HIP library and the
CPU oracle can both be fed from it without sharing any of the method's
arithmetic.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    draft_proposals,
    generate,
    speculative_inputs,
    target_logits,
)
