"""Seeded synthetic inputs for speculative-sampling verification.

This package draws random logits, draft tokens, temperatures, uniforms and
candidate trees. It holds none of the verification arithmetic (no softmax, no
acceptance test, no residual, no argmax over a verified distribution): both the
HIP path and the CPU oracle consume what it produces, and neither is imported
here.
"""
from .synth import (  # noqa: F401
    SEED_BASE,
    ChainConfig,
    TreeConfig,
    CHAIN_CONFIGS,
    TREE_CONFIGS,
    SampleTreeConfig,
    SAMPLE_TREE_CONFIGS,
    sample_tree_inputs,
    MC_CONFIG,
    seed_stream,
    chain_inputs,
    chain_uniforms,
    chain_temperatures,
    mc_chain_inputs,
    sample_inputs,
    tree_parents_ranked,
    tree_inputs,
    sample_draft_tokens_gumbel,
    LMHeadConfig,
    LM_HEAD_CONFIGS,
    lm_head_chain_inputs,
)
