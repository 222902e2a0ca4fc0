"""sv_verify_chain_noalloc: the chain call on the library's static per-GPU
scratch array (no workspace, nothing allocated by the library).

Two calls in a row through the C ABI, the second with a smaller input (the
array keeps the first call's contents, which the second must not see), each
checked bit for bit against sv_verify_chain on the same inputs and against
the oracle (tokens exact outside the flag window, probabilities to 1e-5),
plus the oversize rejection. Every case prints its name before touching the
GPU.
"""
import numpy as np
import pytest
import torch

from parity import assert_chain_parity, compare_chain, oracle_chain
from workloads import CHAIN_CONFIGS, chain_inputs

pytestmark = pytest.mark.gpu

KEYS = ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass", "err_flags")


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _both(sv, inp):
    args = (inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"], inp["uniforms"])
    a = sv.sv_verify_chain_noalloc(*args)
    torch.cuda.synchronize()
    b = sv.sv_verify_chain(*args)
    torch.cuda.synchronize()
    return a, b


def test_two_calls_in_a_row_match_the_workspace_call(sv):
    big = CHAIN_CONFIGS["c2"]
    small = CHAIN_CONFIGS["c1"].with_(B=9, K=3, V=20000, dtype="bf16", variant=57)
    for label, cfg in (("first call, c2 shape", big), ("second call, smaller", small)):
        _say("no-alloc chain call:", label, cfg.name, (cfg.B, cfg.K, cfg.V, cfg.dtype))
        inp = chain_inputs(cfg, device="cuda")
        a, b = _both(sv, inp)
        assert int(a["err_flags"].item()) == 0
        for k in KEYS:
            assert torch.equal(a[k], b[k]), f"{label}: {k} differs from sv_verify_chain"
        assert_chain_parity(compare_chain(a, oracle_chain(inp)))


def test_oversize_is_rejected(sv):
    # B=256, K=63, V=256000 bf16 needs 12.9 MiB of workspace, more than the array
    B, K, V = 256, 63, 256000
    _say("no-alloc oversize rejection", (B, K, V))
    lib = sv.library()
    need = sv.sv_chain_workspace_bytes(B, K, V, torch.bfloat16)
    assert need > 8 << 20
    st = lib.sv_verify_chain_noalloc(None, None, 1, None, None, None, B, K, V, None, None, None, None, None, None,
                                     None, None)
    assert sv.sv_status_string(st) in ("SV_ERR_UNSUPPORTED", "SV_ERR_INVALID_ARGUMENT")
    assert sv.sv_status_string(st) == "SV_ERR_INVALID_ARGUMENT"  # accept_len NULL is checked first
    dummy = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = lib.sv_verify_chain_noalloc(None, None, 1, None, None, None, B, K, V, dummy.data_ptr(), None, None, None,
                                     None, None, None, None)
    assert sv.sv_status_string(st) == "SV_ERR_UNSUPPORTED"
