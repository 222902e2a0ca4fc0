"""The workspace contract on the GPU: one zero-filled workspace serves any
sequence of chain and tree calls, and every successful call leaves it all
zero again (chunked and segment layouts, data-error rows, K = 0, a tree call
in between), with every result still matching the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import assert_chain_parity, compare_chain, oracle_chain
from workloads import CHAIN_CONFIGS, chain_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _chain_case(B, K, V, dtype, seed, bad_token_row=None):
    cfg = CHAIN_CONFIGS["c1"].with_(B=B, K=K, V=V, dtype=dtype, variant=seed)
    inp = chain_inputs(cfg, device="cuda")
    if bad_token_row is not None and K > 0:
        inp["draft_tokens"][bad_token_row, 0] = V
    return inp


def test_workspace_returns_to_zero(sv):
    cases = [
        ("chunked bf16", dict(B=8, K=5, V=4096, dtype="bf16", seed=401)),
        ("segments bf16 (odd V)", dict(B=6, K=3, V=5003, dtype="bf16", seed=402)),
        ("chunked f32 with a bad-token row", dict(B=5, K=4, V=2000, dtype="f32", seed=403, bad_token_row=2)),
        ("K = 0", dict(B=4, K=0, V=3000, dtype="bf16", seed=404)),
        ("segments f32 (V = 33)", dict(B=3, K=2, V=33, dtype="f32", seed=405)),
    ]
    nbytes = max(sv.sv_chain_workspace_bytes(c["B"], c["K"], c["V"], torch.bfloat16 if c["dtype"] == "bf16"
                                             else torch.float32) for _, c in cases)
    nbytes = max(nbytes, sv.sv_tree_workspace_bytes(4, 20, 1000, torch.bfloat16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for round_ in range(2):
        for label, c in cases:
            _say("workspace round", round_, label)
            inp = _chain_case(**c)
            out = sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                                     inp["uniforms"], workspace_tensor=ws)
            torch.cuda.synchronize()
            assert int(ws.count_nonzero().item()) == 0, f"workspace dirty after {label}"
            bad = c.get("bad_token_row")
            flags = int(out["err_flags"].item())
            if bad is None:
                assert flags == 0
                rep = compare_chain(out, oracle_chain(inp))
                assert_chain_parity(rep)
            else:
                assert flags & sv.SV_ERRF_TOKEN
                acc = out["accept_len"].cpu().numpy()
                assert acc[bad] == -1 and np.all(np.delete(acc, bad) >= 0)
        # a tree call on the same workspace
        _say("workspace round", round_, "tree")
        rng = np.random.Generator(np.random.Philox(406))
        N, V, B = 20, 1000, 4
        parents = np.array([-1 if i == 0 or rng.random() < 0.2 else int(rng.integers(0, i)) for i in range(N)],
                           dtype=np.int32)
        target = torch.from_numpy(rng.standard_normal((B, N + 1, V))).to(torch.bfloat16)
        tokens = np.ascontiguousarray(target.float().numpy().argmax(-1)[:, np.where(parents < 0, 0, parents + 1)]
                                      .astype(np.int32))
        out = sv.sv_verify_tree_greedy(target.cuda(), torch.from_numpy(tokens).cuda(),
                                       torch.from_numpy(parents).cuda(), workspace_tensor=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, "workspace dirty after the tree call"
        ref = oracle.verify_tree_greedy(target.float().numpy(), tokens, parents)
        np.testing.assert_array_equal(out["accept_len"].cpu().numpy(), ref["accept_len"])
        np.testing.assert_array_equal(out["next_token"].cpu().numpy(), ref["next_token"])


def test_sampling_leaves_the_workspace_zero(sv):
    # draft-side sampling on a shared workspace, including a bad-temperature row
    rng = np.random.Generator(np.random.Philox(407))
    R, V = 40, 6000
    ws = torch.zeros(sv.sv_sample_workspace_bytes(R, V, torch.bfloat16), dtype=torch.uint8, device="cuda")
    for label, bad in (("clean rows", None), ("a row with T = 0", 3)):
        _say("sampling workspace:", label)
        logits = torch.from_numpy(rng.normal(0, 2, (R, V)).astype(np.float32)).to(torch.bfloat16).cuda()
        T = torch.full((R,), 0.9, device="cuda")
        if bad is not None:
            T[bad] = 0.0
        u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
        out = sv.sv_sample_rows(logits, T, u, workspace_tensor=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, f"workspace dirty after {label}"
        tok = out["tokens"].cpu().numpy()
        if bad is None:
            assert int(out["err_flags"].item()) == 0
            ref, _, lo, hi = oracle.sample_rows(logits.float().cpu().numpy(), T.cpu().numpy(), u.cpu().numpy())
            uu = u.double().cpu().numpy()
            near = (np.abs(uu - lo) < oracle.FLAG_WINDOW) | (np.abs(hi - uu) < oracle.FLAG_WINDOW)
            assert np.array_equal(tok[~near], ref[~near]), np.nonzero((tok != ref) & ~near)[0]
        else:
            assert int(out["err_flags"].item()) & sv.SV_ERRF_TEMPERATURE
            assert tok[bad] == -1 and np.all(np.delete(tok, bad) >= 0)


def test_sampling_workspace_across_shapes(sv):
    # one workspace, sized for the largest, serves draft-side sampling calls
    # of very different unit counts back to back (the groups' counters and
    # the records are all zero after each call)
    shapes = [(5000, 8), (320, 12800), (3, 128256), (5000, 8)]
    nbytes = max(sv.sv_sample_workspace_bytes(R, V, torch.bfloat16) for R, V in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    rng = np.random.Generator(np.random.Philox(409))
    for R, V in shapes:
        _say("sampling workspace across shapes: R =", R, "V =", V)
        logits = torch.from_numpy(rng.normal(0, 2, (R, V)).astype(np.float32)).to(torch.bfloat16).cuda()
        T = torch.full((R,), 0.8, device="cuda")
        u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
        out = sv.sv_sample_rows(logits, T, u, workspace_tensor=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, f"workspace dirty after R={R} V={V}"
        assert int(out["err_flags"].item()) == 0
        ref, _, lo, hi = oracle.sample_rows(logits.float().cpu().numpy(), T.cpu().numpy(), u.cpu().numpy())
        uu = u.double().cpu().numpy()
        near = (np.abs(uu - lo) < oracle.FLAG_WINDOW) | (np.abs(hi - uu) < oracle.FLAG_WINDOW)
        tok = out["tokens"].cpu().numpy()
        assert np.array_equal(tok[~near], ref[~near]), np.nonzero((tok != ref) & ~near)[0]


def test_one_launch_call_leaves_the_workspace_zero(sv):
    # calls whose grid is larger than the device holds at once take the
    # one-launch kernel (ticket queues, chunk counters and arrival counters
    # per sequence): one zero-filled workspace serves them back to back, is
    # all zero after each, and a two-launch call on it in between still works
    big = CHAIN_CONFIGS["c2"]
    small = dict(B=8, K=5, V=4096, dtype="bf16", seed=408)
    nbytes = max(sv.sv_chain_workspace_bytes(big.B, big.K, big.V, torch.bfloat16),
                 sv.sv_chain_workspace_bytes(small["B"], small["K"], small["V"], torch.bfloat16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (label, inp) in enumerate([("one-launch c2", chain_inputs(big, device="cuda")),
                                      ("two-launch B8", _chain_case(**small)),
                                      ("one-launch c2, second input set",
                                       chain_inputs(big.with_(variant=big.variant + 10), device="cuda"))]):
        _say("workspace:", label)
        out = sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                                 inp["uniforms"], workspace_tensor=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, f"workspace dirty after {label}"
        assert int(out["err_flags"].item()) == 0
        assert_chain_parity(compare_chain(out, oracle_chain(inp)))
