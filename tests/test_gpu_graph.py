"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

A call allocates nothing, records no memset and leaves its workspace all zero,
so a captured call can be replayed. Each test captures one call with every
output and the workspace allocated beforehand, replays the graph several
times with other eager work (other inputs, other workspaces) in between, and
checks every replay bit for bit against the eager call on the same inputs.
"""
import pytest
import torch

from workloads import (CHAIN_CONFIGS, SAMPLE_TREE_CONFIGS, TREE_CONFIGS, chain_inputs, sample_inputs,
                       sample_tree_inputs, tree_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _replay_and_compare(g, outs, ref, other):
    for rep in range(4):
        for k, t in outs.items():
            if k != "err_flags":
                t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(outs[k], ref[k]), f"replay {rep}: {k} differs from the eager call"
        other()  # eager work between replays
        torch.cuda.synchronize()


def test_chain_call_in_a_graph(sv):
    cfg = CHAIN_CONFIGS["c2"]
    _say("graph: chain", cfg.name)
    inp = chain_inputs(cfg, device="cuda")
    alt = chain_inputs(cfg.with_(variant=cfg.variant + 10), device="cuda")
    args = [inp[k] for k in ("target", "draft", "draft_tokens", "temperature", "uniforms")]
    ref = sv.sv_verify_chain(*args, want_entropy=True)
    torch.cuda.synchronize()
    B, K1, V = inp["target"].shape
    outs = {"accept_len": torch.empty(B, dtype=torch.int32, device="cuda"),
            "out_tokens": torch.empty(B, K1, dtype=torch.int32, device="cuda"),
            "p_draft": torch.empty(B, K1 - 1, device="cuda"), "q_draft": torch.empty(B, K1 - 1, device="cuda"),
            "residual_mass": torch.empty(B, device="cuda"), "entropy": torch.empty(B, 2 * K1 - 1, device="cuda"),
            "err_flags": torch.zeros(1, dtype=torch.int32, device="cuda")}
    ws = torch.zeros(sv.sv_chain_workspace_bytes(B, K1 - 1, V, inp["target"].dtype), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # one call on the capture stream before capturing
        sv.sv_verify_chain(*args, workspace_tensor=ws, **outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sv.sv_verify_chain(*args, workspace_tensor=ws, **outs)
    alt_args = [alt[k] for k in ("target", "draft", "draft_tokens", "temperature", "uniforms")]
    _replay_and_compare(g, outs, {k: v for k, v in ref.items()}, lambda: sv.sv_verify_chain(*alt_args))
    assert int(outs["err_flags"].item()) == 0


def test_sampling_call_in_a_graph(sv):
    cfg = CHAIN_CONFIGS["c2"]
    _say("graph: draft-side sampling over the draft rows of", cfg.name)
    inp = sample_inputs(cfg, device="cuda")
    ref = sv.sv_sample_rows(inp["logits"], inp["temperature"], inp["uniforms"])
    torch.cuda.synchronize()
    R, V = inp["logits"].shape
    outs = {"tokens": torch.empty(R, dtype=torch.int32, device="cuda"), "prob": torch.empty(R, device="cuda"),
            "err_flags": torch.zeros(1, dtype=torch.int32, device="cuda")}
    ws = torch.zeros(sv.sv_sample_workspace_bytes(R, V, inp["logits"].dtype), dtype=torch.uint8, device="cuda")

    def call():
        sv.sv_sample_rows(inp["logits"], inp["temperature"], inp["uniforms"], out_tokens=outs["tokens"],
                          out_prob=outs["prob"], err_flags=outs["err_flags"], workspace_tensor=ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    _replay_and_compare(g, outs, {"tokens": ref["tokens"], "prob": ref["prob"]},
                        lambda: sv.sv_sample_rows(inp["logits"], None, inp["uniforms"]))


def test_tree_call_in_a_graph(sv):
    cfg = TREE_CONFIGS["c4"].with_(B=8)
    _say("graph: greedy tree", cfg.name, "B = 8")
    inp = tree_inputs(cfg, device="cuda")
    ref = sv.sv_verify_tree_greedy(inp["target"], inp["node_tokens"], inp["parents"])
    torch.cuda.synchronize()
    B, N1, V = inp["target"].shape
    N = N1 - 1
    outs = {"accept_len": torch.empty(B, dtype=torch.int32, device="cuda"),
            "path_nodes": torch.empty(B, N, dtype=torch.int32, device="cuda"),
            "next_token": torch.empty(B, dtype=torch.int32, device="cuda"),
            "err_flags": torch.zeros(1, dtype=torch.int32, device="cuda")}
    ws = torch.zeros(sv.sv_tree_workspace_bytes(B, N, V, inp["target"].dtype), dtype=torch.uint8, device="cuda")

    def call():
        sv.sv_verify_tree_greedy(inp["target"], inp["node_tokens"], inp["parents"], workspace_tensor=ws, **outs)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    _replay_and_compare(g, outs, {k: ref[k] for k in ("accept_len", "path_nodes", "next_token")},
                        lambda: sv.sv_verify_tree_greedy(inp["target"], inp["node_tokens"], inp["parents"]))


def test_tree_sampling_call_in_a_graph(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(B=8)
    _say("graph: sampling tree", cfg.name, "B = 8")
    inp = sample_tree_inputs(cfg, device="cuda")
    keys = ("target", "draft", "node_tokens", "parents", "temperature", "uniforms")
    ref = sv.sv_verify_tree_sampling(*(inp[k] for k in keys))
    torch.cuda.synchronize()
    B, N1, V = inp["target"].shape
    N = N1 - 1
    outs = {"accept_len": torch.empty(B, dtype=torch.int32, device="cuda"),
            "path_nodes": torch.empty(B, N, dtype=torch.int32, device="cuda"),
            "next_token": torch.empty(B, dtype=torch.int32, device="cuda"),
            "err_flags": torch.zeros(1, dtype=torch.int32, device="cuda")}
    ws = torch.zeros(sv.sv_tree_sampling_workspace_bytes(B, N, V, inp["target"].dtype), dtype=torch.uint8,
                     device="cuda")

    def call():
        sv.sv_verify_tree_sampling(*(inp[k] for k in keys), workspace_tensor=ws, **outs)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    alt = sample_tree_inputs(cfg.with_(variant=cfg.variant + 10), device="cuda")
    _replay_and_compare(g, outs, {k: ref[k] for k in ("accept_len", "path_nodes", "next_token")},
                        lambda: sv.sv_verify_tree_sampling(*(alt[k] for k in keys)))
    assert int(outs["err_flags"].item()) == 0
