"""Calls on a stream that is not the current one.

The binding allocates and zero-fills outputs, err_flags and cached workspaces
for a call; all of that has to be ordered before the call's kernels on the
call's stream. These tests pass ``stream=s`` from outside any
``torch.cuda.stream(s)`` block, on workspace keys no earlier call used, while
the caller's current stream is still busy with a long (bounded) spin kernel,
and on memory the caching allocator last handed out filled with 0xff bytes.
Every result must match the oracle as in the parity tests, and no error bit
may be raised. Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import assert_chain_parity, compare_chain, oracle_chain
from workloads import CHAIN_CONFIGS, SAMPLE_TREE_CONFIGS, chain_inputs, sample_tree_inputs

pytestmark = pytest.mark.gpu

# about 20 ms of spinning at a 100 MHz-class clock count: long enough that a
# zero-fill queued behind it would still be pending when the call's kernels run
_SPIN_CYCLES = 50_000_000


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _dirty_allocator(nbytes: int) -> None:
    """Leave freed blocks full of 0xff in the caching allocator (a later
    allocation of this size class may reuse them without clearing)."""
    junk = torch.full((nbytes,), 0xff, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    del junk


def _busy_current_stream() -> None:
    torch.cuda._sleep(_SPIN_CYCLES)


def test_chain_on_another_stream(sv):
    cfg = CHAIN_CONFIGS["c1"].with_(B=48, K=5, V=20000, dtype="bf16", variant=31)
    _say("chain on a side stream", cfg.name, "B48 K5 V20000 bf16 variant 31")
    inp = chain_inputs(cfg, device="cuda")
    _dirty_allocator(64 << 20)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    _busy_current_stream()
    out = sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"], inp["uniforms"],
                             stream=s)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    assert_chain_parity(compare_chain(out, oracle_chain(inp)))


def test_prepared_chain_on_another_stream(sv):
    cfg = CHAIN_CONFIGS["c1"].with_(B=40, K=4, V=12000, dtype="bf16", variant=32)
    _say("prepared chain call on a side stream", cfg.name, "B40 K4 V12000 bf16 variant 32")
    inp = chain_inputs(cfg, device="cuda")
    _dirty_allocator(64 << 20)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    _busy_current_stream()
    call = sv.PreparedChainCall(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                                inp["uniforms"], stream=s)
    for _ in range(3):
        out = call()
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    assert_chain_parity(compare_chain(out, oracle_chain(inp)))


def test_tree_sampling_on_another_stream(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(B=6, N=20, V=4096)
    _say("sampling tree on a side stream", cfg.name, "B6 N20 V4096")
    inp = sample_tree_inputs(cfg, device="cuda")
    _dirty_allocator(64 << 20)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    _busy_current_stream()
    out = sv.sv_verify_tree_sampling(inp["target"], inp["draft"], inp["node_tokens"], inp["parents"],
                                     inp["temperature"], inp["uniforms"], stream=s)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    np_ = lambda t: t.detach().cpu().numpy()
    ref = oracle.verify_tree_stochastic(np_(inp["target"].double()), np_(inp["draft"].double()),
                                        np_(inp["node_tokens"]).astype(np.int64), np_(inp["parents"]).astype(np.int64),
                                        np_(inp["temperature"]).astype(np.float64),
                                        np_(inp["uniforms"]).astype(np.float64))
    ok = ~ref["flagged"]
    assert np.array_equal(np_(out["accept_len"])[ok], ref["accept_len"][ok])
    assert np.array_equal(np_(out["path_nodes"])[ok], ref["path_nodes"][ok])
    assert np.array_equal(np_(out["next_token"])[ok], ref["next_token"][ok])


def test_sample_rows_on_another_stream(sv):
    rng = np.random.Generator(np.random.Philox(33))
    R, V = 24, 8192
    _say("draft-side sampling on a side stream", f"R{R} V{V} bf16 seed 33")
    logits = torch.from_numpy(rng.normal(0, 2.0, (R, V))).to(torch.bfloat16).cuda()
    T = torch.from_numpy(rng.uniform(0.5, 1.5, R).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    _dirty_allocator(64 << 20)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    _busy_current_stream()
    out = sv.sv_sample_rows(logits, T, u, stream=s)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    tok, _, lo, hi = oracle.sample_rows(logits.double().cpu().numpy(), T.double().cpu().numpy(),
                                        u.double().cpu().numpy())
    uu = u.double().cpu().numpy()
    ok = ~((np.abs(uu - lo) < oracle.FLAG_WINDOW) | (np.abs(hi - uu) < oracle.FLAG_WINDOW))
    assert np.array_equal(out["tokens"].cpu().numpy()[ok], tok[ok])
