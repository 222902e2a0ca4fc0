"""GPU parity of sv_verify_tree_greedy and sv_build_tree_mask against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import record_parity
from workloads import TREE_CONFIGS, tree_inputs, tree_parents_ranked

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _tree_parity(sv, target, tokens, parents, label):
    _say(label, tuple(target.shape), target.dtype, "N", parents.numel())
    out = sv.sv_verify_tree_greedy(target, tokens, parents)
    torch.cuda.synchronize()
    ref = oracle.verify_tree_greedy(_np(target.float()), _np(tokens), _np(parents))
    np.testing.assert_array_equal(_np(out["accept_len"]), ref["accept_len"])
    np.testing.assert_array_equal(_np(out["path_nodes"]), ref["path_nodes"])
    np.testing.assert_array_equal(_np(out["next_token"]), ref["next_token"])
    return out, ref


def test_c4_full(sv):
    cfg = TREE_CONFIGS["c4"]
    inp = tree_inputs(cfg, device="cuda")
    out, ref = _tree_parity(sv, inp["target"], inp["node_tokens"], inp["parents"], cfg.name)
    assert int(out["err_flags"].item()) == 0
    mean_len = ref["accept_len"].mean()
    print(cfg.name, "mean accept_len", mean_len, flush=True)
    assert 0.5 < mean_len < 4.0
    # argmax ties at bf16 happen in this workload; the lowest id must win
    g = ref["argmax"]
    t = _np(inp["target"].float())
    ties = sum(int((t[b, n] == t[b, n, g[b, n]]).sum() > 1) for b in range(cfg.B) for n in range(cfg.N + 1))
    print(cfg.name, "positions with a tied maximum:", ties, flush=True)
    mask = sv.sv_build_tree_mask(inp["parents"])
    torch.cuda.synchronize()
    mask_same = bool(np.array_equal(_np(mask["mask"]), oracle.tree_mask(_np(inp["parents"]))))
    assert mask_same
    record_parity(cfg.name, call="sv_verify_tree_greedy + sv_build_tree_mask", rows=cfg.B,
                  mismatched=int((_np(out["accept_len"]) != ref["accept_len"]).sum()
                                 + (_np(out["path_nodes"]) != ref["path_nodes"]).any(axis=1).sum()
                                 + (_np(out["next_token"]) != ref["next_token"]).sum()),
                  positions_with_tied_maximum=ties, mask_bit_exact=mask_same,
                  mask_bytes=int(cfg.N * cfg.N), mean_accept_len=float(mean_len))


def _random_tree(rng, N, p_root=0.15):
    return np.array([-1 if i == 0 or rng.random() < p_root else int(rng.integers(0, i)) for i in range(N)],
                    dtype=np.int32)


CASES = [
    (4, 1, 3, torch.float32),
    (8, 2, 1000, torch.bfloat16),
    (8, 7, 32003, torch.bfloat16),
    (8, 64, 5000, torch.float32),
    (8, 65, 5000, torch.bfloat16),
    (4, 200, 3001, torch.bfloat16),
    (2, 1024, 700, torch.bfloat16),
]


@pytest.mark.parametrize("B,N,V,dtype", CASES, ids=[f"B{b}_N{n}_V{v}_{str(d)[6:]}" for b, n, v, d in CASES])
def test_random_trees(sv, B, N, V, dtype):
    rng = np.random.Generator(np.random.Philox(300 + N + V))
    parents = _random_tree(rng, N)
    target = torch.from_numpy(rng.standard_normal((B, N + 1, V)) * 3).to(dtype)
    g = target.float().numpy().argmax(-1)
    pos = np.where(parents < 0, 0, parents + 1)
    tokens = np.ascontiguousarray(
        np.where(rng.random((B, N)) < 0.8, g[:, pos], rng.integers(0, V, (B, N))).astype(np.int32))
    _tree_parity(sv, target.cuda(), torch.from_numpy(tokens).cuda(), torch.from_numpy(parents).cuda(),
                 f"random tree B{B} N{N} V{V}")


@pytest.mark.parametrize("N", [64, 1024])
def test_chain_shaped_deep_tree(sv, N):
    """A chain of N nodes: depth N (all pointer-jumping rounds), cut at several depths."""
    B, V = 4, 64
    rng = np.random.Generator(np.random.Philox(310 + N))
    parents = np.arange(-1, N - 1, dtype=np.int32)
    target = torch.from_numpy(rng.standard_normal((B, N + 1, V))).float()
    g = target.numpy().argmax(-1)
    tokens = g[:, :N].copy().astype(np.int32)
    cuts = [N, N - 24, 3, 0]
    for b, c in enumerate(cuts):
        if c < N:
            tokens[b, c] = (g[b, c] + 1) % V
    out, ref = _tree_parity(sv, target.cuda(), torch.from_numpy(tokens).cuda(), torch.from_numpy(parents).cuda(),
                            f"chain-shaped tree N{N}")
    np.testing.assert_array_equal(_np(out["accept_len"]), cuts)


def test_star_tree_accepts_at_most_one(sv):
    B, N, V = 6, 64, 500
    rng = np.random.Generator(np.random.Philox(313))
    parents = np.full(N, -1, dtype=np.int32)
    target = torch.from_numpy(rng.standard_normal((B, N + 1, V)) * 2).to(torch.bfloat16)
    g = target.float().numpy().argmax(-1)
    tokens = rng.integers(0, V, (B, N)).astype(np.int32)
    tokens[:3, 17] = g[:3, 0]   # a child of the root that matches
    tokens[:2, 40] = g[:2, 0]   # a second matching child: the lower id wins
    out, ref = _tree_parity(sv, target.cuda(), torch.from_numpy(tokens).cuda(), torch.from_numpy(parents).cuda(),
                            "star tree N64")
    assert np.all(ref["accept_len"] <= 1)


def test_argmax_ties_lowest_id(sv):
    B, N, V = 16, 30, 3000
    rng = np.random.Generator(np.random.Philox(311))
    parents = _random_tree(rng, N)
    # integer logits in a small range: many tied maxima per row
    target = torch.from_numpy(rng.integers(-3, 4, (B, N + 1, V)).astype(np.float32)).to(torch.bfloat16)
    g = target.float().numpy().argmax(-1)
    pos = np.where(parents < 0, 0, parents + 1)
    tokens = np.ascontiguousarray(g[:, pos].astype(np.int32))
    out, ref = _tree_parity(sv, target.cuda(), torch.from_numpy(tokens).cuda(), torch.from_numpy(parents).cuda(),
                            "ties")
    assert np.all(ref["accept_len"] > 0)


def test_tree_data_errors(sv):
    B, N, V = 4, 6, 100
    rng = np.random.Generator(np.random.Philox(312))
    target = torch.from_numpy(rng.standard_normal((B, N + 1, V))).float().cuda()
    parents = torch.tensor([-1, 0, 0, 1, 1, 2], dtype=torch.int32, device="cuda")
    tokens = torch.from_numpy(rng.integers(0, V, (B, N)).astype(np.int32)).cuda()
    tokens[2, 3] = V
    _say("tree token error")
    out = sv.sv_verify_tree_greedy(target, tokens, parents)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) & sv.SV_ERRF_TOKEN
    assert _np(out["accept_len"])[2] == -1 and np.all(_np(out["path_nodes"])[2] == -1)
    assert np.all(_np(out["accept_len"])[[0, 1, 3]] >= 0)
    bad_par = torch.tensor([-1, 0, 2, 1, 1, 2], dtype=torch.int32, device="cuda")
    _say("tree parent error")
    out = sv.sv_verify_tree_greedy(target, tokens, bad_par)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) & sv.SV_ERRF_PARENT
    assert np.all(_np(out["accept_len"]) == -1)


# ----------------------------------------------------------------------------- mask

@pytest.mark.parametrize("N", [1, 6, 64, 65, 200, 1024])
def test_mask_matches_oracle(sv, N):
    rng = np.random.Generator(np.random.Philox(320 + N))
    parents = _random_tree(rng, N)
    _say("mask N", N)
    out = sv.sv_build_tree_mask(torch.from_numpy(parents).cuda())
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    np.testing.assert_array_equal(_np(out["mask"]), oracle.tree_mask(parents))


def test_mask_of_the_workload_tree(sv):
    parents, _ = tree_parents_ranked((4, 3, 2, 2, 1), 64)
    _say("mask of the 64-node ranked tree")
    out = sv.sv_build_tree_mask(torch.from_numpy(parents).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(out["mask"]), oracle.tree_mask(parents))


def test_mask_bad_parent(sv):
    _say("mask parent error")
    out = sv.sv_build_tree_mask(torch.tensor([-1, 0, 5, 1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) & sv.SV_ERRF_PARENT
