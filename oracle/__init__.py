"""CPU oracle for speculative-sampling verification — test infrastructure only.

Imported by the test suite, the smoke check and the benchmark's CPU-baseline leg;
never by the product library or its binding.
"""
from .specverify_oracle import (  # noqa: F401
    FLAG_WINDOW,
    temperature_softmax,
    entropy,
    acceptance_probability,
    residual_weights,
    inverse_cdf,
    sample_rows,
    verify_chain,
    verify_chain_distributions,
    chain_rows_valid,
    node_depths,
    verify_tree_greedy,
    verify_tree_stochastic,
    children_in_order,
    tree_mask,
    round_to_bf16,
    lm_head_logits,
    verify_chain_lm_head,
)
