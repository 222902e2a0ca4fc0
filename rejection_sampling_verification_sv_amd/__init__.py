"""specverify for AMD MI355X: speculative-sampling verification in HIP.

The compute lives in ``libspecverify.so`` (HIP kernels for gfx950 behind a C
ABI declared in ``include/specverify.h``); :mod:`.specverify` is its thin
ctypes binding. Build with ``python -m rejection_sampling_verification_sv_amd.build``.
"""
from .specverify import (  # noqa: F401
    PreparedChainCall,
    PreparedLMHeadChainCall,
    PreparedLMHeadLogitsCall,
    PreparedSampleCall,
    PreparedTreeCall,
    PreparedTreeSamplingCall,
    SpecVerifyError,
    SV_DTYPE_BF16,
    SV_DTYPE_F32,
    SV_ERRF_INTERNAL,
    SV_ERRF_NONFINITE,
    SV_ERRF_PARENT,
    SV_ERRF_TEMPERATURE,
    SV_ERRF_TOKEN,
    SV_MAX_K,
    SV_MAX_TREE_NODES,
    library,
    reset_workspaces,
    sv_build_tree_mask,
    sv_chain_form,
    sv_chain_launches,
    sv_chain_workspace_bytes,
    sv_sample_rows,
    sv_sample_workspace_bytes,
    sv_status_string,
    sv_time_next_stream_pass,
    sv_tree_sampling_workspace_bytes,
    sv_tree_workspace_bytes,
    sv_verify_chain,
    sv_verify_chain_noalloc,
    sv_verify_chain_lm_head,
    sv_lm_head_logits,
    sv_lm_head_chain_workspace_bytes,
    sv_verify_tree_greedy,
    sv_verify_tree_sampling,
)
