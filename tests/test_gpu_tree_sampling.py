"""GPU parity of sv_verify_tree_sampling against the oracle's sampling tree verification.

Bar: accept_len, path_nodes and next_token bit-exact per sequence, except
sequences the oracle flags (a tested uniform, or the final one against a CDF
boundary of the drawn token, within 1e-6 of its threshold); flagged sequences
are counted and printed. A sequence whose only flag is the final draw must
still match in accept_len and path_nodes. Losslessness on the GPU is checked
by Monte Carlo: the first emitted token follows the target's distribution at
the root, and, given that child v was accepted first, the next emitted token
follows the target's distribution at v's position.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import record_parity
from workloads import SAMPLE_TREE_CONFIGS, sample_draft_tokens_gumbel, sample_tree_inputs, seed_stream

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


def _oracle(inp, b0=0, b1=None, per=4):
    """The oracle on sequences [b0, b1), a few sequences at a time (fp64 copies stay small)."""
    B = inp["target"].shape[0]
    b1 = B if b1 is None else b1
    parts = []
    for s0 in range(b0, b1, per):
        s1 = min(b1, s0 + per)
        T = inp["temperature"]
        T = np.ones(s1 - s0) if T is None else _np(T[s0:s1]).astype(np.float64)
        parts.append(oracle.verify_tree_stochastic(
            _np(inp["target"][s0:s1].double()), _np(inp["draft"][s0:s1].double()),
            _np(inp["node_tokens"][s0:s1]).astype(np.int64), _np(inp["parents"]).astype(np.int64), T,
            _np(inp["uniforms"][s0:s1]).astype(np.float64)))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def _call(sv, inp, **kw):
    out = sv.sv_verify_tree_sampling(inp["target"], inp["draft"], inp["node_tokens"], inp["parents"],
                                     inp["temperature"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    return out


def _compare(out, ref, label):
    acc = _np(out["accept_len"]).astype(np.int64)
    path = _np(out["path_nodes"]).astype(np.int64)
    nxt = _np(out["next_token"]).astype(np.int64)
    same_path = (acc == ref["accept_len"]) & np.all(path == ref["path_nodes"], axis=1)
    same = same_path & (nxt == ref["next_token"])
    flagged = ref["flagged"]
    path_flag = ref["margin"] < oracle.FLAG_WINDOW
    print(f"{label}: sequences {len(acc)}, flagged {int(flagged.sum())} (path decisions {int(path_flag.sum())}), "
          f"mismatched flagged {int((~same & flagged).sum())}, mean accept_len "
          f"{ref['accept_len'][ref['valid']].mean() if ref['valid'].any() else float('nan'):.3f}, "
          f"children tested {int(ref['tests'].sum())}", flush=True)
    bad = ~same & ~flagged
    assert not bad.any(), (label, np.nonzero(bad)[0][:8], acc[bad][:8], ref["accept_len"][bad][:8],
                           nxt[bad][:8], ref["next_token"][bad][:8])
    bad_path = ~same_path & ~path_flag
    assert not bad_path.any(), (label, np.nonzero(bad_path)[0][:8])
    return same


def _structure(out, parents, N, V):
    acc = _np(out["accept_len"]).astype(np.int64)
    path = _np(out["path_nodes"]).astype(np.int64)
    nxt = _np(out["next_token"]).astype(np.int64)
    ok = acc >= 0
    assert np.all(acc[ok] <= N)
    assert np.all((nxt[ok] >= 0) & (nxt[ok] < V))
    assert np.all(nxt[~ok] == -1) and np.all(path[~ok] == -1)
    for b in np.nonzero(ok)[0]:
        d = acc[b]
        assert np.all(path[b, d:] == -1)
        prev = -1
        for v in path[b, :d]:
            assert parents[v] == prev
            prev = v


def test_c4s_full(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"]
    _say(cfg.name)
    inp = sample_tree_inputs(cfg, device="cuda")
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == 0
    ref = _oracle(inp)
    assert ref["valid"].all()
    same = _compare(out, ref, cfg.name)
    _structure(out, _np(inp["parents"]), cfg.N, cfg.V)
    record_parity(cfg.name, call="sv_verify_tree_sampling", rows=cfg.B, flagged=int(ref["flagged"].sum()),
                  mismatched_unflagged=int((~same & ~ref["flagged"]).sum()),
                  mismatched_flagged=int((~same & ref["flagged"]).sum()),
                  min_margin=float(ref["margin"].min()), mean_accept_len=float(ref["accept_len"].mean()),
                  children_tested=int(ref["tests"].sum()))
    assert 0.5 < ref["accept_len"].mean() < 5.0


def _random_tree(rng, N, p_root=0.2):
    return np.array([-1 if i == 0 or rng.random() < p_root else int(rng.integers(0, i)) for i in range(N)],
                    dtype=np.int32)


# (B, N, V, dtype, sigma_t, sigma_d, T): rows of 1 run, a ragged last run, more
# runs than the walk's 16 waves, more than 64 runs (the draw's scan loops)
CASES = [
    (6, 1, 8, "bf16", 2.0, 1.0, 1.0),
    (16, 12, 1000, "f32", 1.0, 1.5, 1.0),
    (24, 30, 5000, "bf16", 2.0, 2.0, 0.7),
    (12, 20, 2052, "f32", 3.0, 1.0, 1.3),
    (8, 40, 40000, "bf16", 2.5, 1.5, 1.0),
    (6, 16, 70000, "bf16", 3.0, 2.0, 0.9),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_N{c[1]}_V{c[2]}_{c[3]}" for c in CASES])
def test_random_trees(sv, case):
    B, N, V, dt, st, sd, T = case
    rng = seed_stream(91, N * 7 + V % 97, 0)
    parents = _random_tree(rng, N)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name=f"tree_sampling_random_b{B}_n{N}_v{V}", B=B, N=N, V=V, dtype=dt,
                                           target_sigma=st, draft_sigma=sd, temperature=T, variant=N + V)
    _say(cfg.name, dt, "parents", parents.tolist()[:12])
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == 0
    ref = _oracle(inp)
    _compare(out, ref, cfg.name)
    _structure(out, parents, N, V)


def test_bushy_and_star_trees(sv):
    # many siblings at one node: up to 31 rejections before the draw
    for parents, label in (([-1] * 32, "star32"), ([-1] * 8 + [0] * 8 + [8] * 8, "two levels of 8")):
        parents = np.array(parents, dtype=np.int32)
        N = len(parents)
        cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name=f"tree_sampling_{label}", B=32, N=N, V=3000, dtype="bf16",
                                               target_sigma=2.0, draft_sigma=2.0, temperature=1.0, variant=N)
        _say(cfg.name)
        inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
        out = _call(sv, inp)
        assert int(out["err_flags"].item()) == 0
        ref = _oracle(inp)
        _compare(out, ref, cfg.name)


def test_chain_tree_matches_chain_call(sv):
    # one child per node: the tree call is chain verification
    B, K, V = 48, 6, 4096
    parents = np.arange(-1, K - 1, dtype=np.int32)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_chain", B=B, N=K, V=V, dtype="bf16",
                                           target_sigma=2.0, draft_sigma=1.5, temperature=1.0, variant=5)
    _say(cfg.name)
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    tree = _call(sv, inp)
    chain = sv.sv_verify_chain(inp["target"], inp["draft"][:, :K].contiguous(), inp["node_tokens"],
                               inp["temperature"], inp["uniforms"])
    torch.cuda.synchronize()
    ref = _oracle(inp)
    same = _compare(tree, ref, cfg.name)
    acc_c = _np(chain["accept_len"]).astype(np.int64)
    out_c = _np(chain["out_tokens"]).astype(np.int64)
    acc_t = _np(tree["accept_len"]).astype(np.int64)
    nxt_t = _np(tree["next_token"]).astype(np.int64)
    agree = (acc_c == acc_t) & (out_c[np.arange(B), acc_c] == nxt_t)
    assert np.all(agree | ref["flagged"]), np.nonzero(~agree)[0]
    print("chain call and tree call agree on", int(agree.sum()), "of", B, "; oracle matches", int(same.sum()))


def test_identical_draft_accepts_first_children(sv):
    # p == q bit for bit: every first child is accepted (alpha = 1), down to a leaf
    parents = np.array([-1, -1, 0, 0, 2, 1, 4, 4, 6], dtype=np.int32)
    N = len(parents)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_identical", B=16, N=N, V=1024, dtype="f32",
                                           variant=3)
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    inp["draft"] = inp["target"].clone()
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == 0
    first_chain = [0, 2, 4, 6, 8]
    assert np.all(_np(out["accept_len"]) == len(first_chain))
    assert np.all(_np(out["path_nodes"])[:, :5] == np.array(first_chain))
    ref = _oracle(inp)
    _compare(out, ref, cfg.name)


def test_max_depth_chain(sv):
    # SV_MAX_TREE_NODES nodes in one chain, p == q: the whole chain is accepted
    N = sv.SV_MAX_TREE_NODES
    parents = np.arange(-1, N - 1, dtype=np.int32)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_max_depth", B=2, N=N, V=256, dtype="bf16", variant=11)
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    inp["draft"] = inp["target"].clone()
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == 0
    assert np.all(_np(out["accept_len"]) == N)
    np.testing.assert_array_equal(_np(out["path_nodes"]), np.tile(np.arange(N), (2, 1)))
    ref = _oracle(inp)
    _compare(out, ref, cfg.name)


def test_max_width_star(sv):
    # SV_MAX_TREE_NODES children of the root (up to 1023 rejections): valid outputs, no error
    N = sv.SV_MAX_TREE_NODES
    parents = np.full(N, -1, dtype=np.int32)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_max_width", B=4, N=N, V=512, dtype="bf16",
                                           target_sigma=1.0, draft_sigma=3.0, variant=12)
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == 0
    _structure(out, parents, N, cfg.V)


def test_max_width_star_split_walk(sv):
    # SV_MAX_TREE_NODES children of the root on long rows: the walk is shared by
    # eight workgroups and exchanges run totals after each of hundreds of
    # rejections (both slot buffers, pass numbers past a thousand)
    N = sv.SV_MAX_TREE_NODES
    parents = np.full(N, -1, dtype=np.int32)
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_max_width_split", B=1, N=N, V=128256, dtype="bf16",
                                           target_sigma=1.0, draft_sigma=3.0, variant=13)
    inp = sample_tree_inputs(cfg, device="cuda", parents=parents)
    ws = torch.zeros(sv.sv_tree_sampling_workspace_bytes(cfg.B, N, cfg.V, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    _say("max-width star, split walk")
    out = _call(sv, inp, workspace_tensor=ws)
    assert int(out["err_flags"].item()) == 0
    assert int(ws.count_nonzero().item()) == 0
    _structure(out, parents, N, cfg.V)
    ref = _oracle(inp)
    print(f"children tested {int(ref['tests'].sum())}", flush=True)
    _compare(out, ref, cfg.name)


def test_temperature_none_is_one(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_t1", B=8, N=10, V=2048, variant=21)
    inp = sample_tree_inputs(cfg, device="cuda")
    a = _call(sv, inp)
    inp2 = dict(inp, temperature=None)
    b = _call(sv, inp2)
    for k in ("accept_len", "path_nodes", "next_token"):
        assert torch.equal(a[k], b[k])


def test_data_errors_per_sequence(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_errors", B=6, N=10, V=2048, variant=31)
    inp = sample_tree_inputs(cfg, device="cuda")
    inp["node_tokens"][1, 7] = cfg.V              # a token outside [0, V)
    inp["temperature"][2] = 0.0                   # an invalid temperature
    inp["target"][3, 0, 5] = float("nan")         # a non-finite root row
    ws = torch.zeros(sv.sv_tree_sampling_workspace_bytes(cfg.B, cfg.N, cfg.V, inp["target"].dtype),
                     dtype=torch.uint8, device="cuda")
    out = _call(sv, inp, workspace_tensor=ws)
    flags = int(out["err_flags"].item())
    assert flags == sv.SV_ERRF_TOKEN | sv.SV_ERRF_TEMPERATURE | sv.SV_ERRF_NONFINITE
    acc = _np(out["accept_len"])
    assert list(acc[1:4]) == [-1, -1, -1]
    assert np.all(_np(out["next_token"])[1:4] == -1)
    good = [0, 4, 5]
    ref = _oracle(inp, 0, 1)
    ref = {k: np.concatenate([ref[k], _oracle(inp, 4, 6)[k]]) for k in ref}
    sub = {k: v[good] for k, v in out.items() if k != "err_flags"}
    _compare(sub, ref, cfg.name)
    # the call leaves its workspace zero, error rows included
    assert int(ws.count_nonzero().item()) == 0


def test_bad_parent(sv):
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_bad_parent", B=3, N=6, V=512, variant=41)
    inp = sample_tree_inputs(cfg, device="cuda")
    inp["parents"] = torch.tensor([-1, 0, 2, 1, 1, 0], dtype=torch.int32, device="cuda")  # 2 is not < 2
    out = _call(sv, inp)
    assert int(out["err_flags"].item()) == sv.SV_ERRF_PARENT
    assert np.all(_np(out["accept_len"]) == -1)
    assert np.all(_np(out["path_nodes"]) == -1)


def test_workspace_reuse_across_shapes(sv):
    big = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_ws_a", B=8, N=20, V=4096, variant=51)
    small = big.with_(name="tree_sampling_ws_b", B=3, N=5, V=1024, dtype="f32", variant=52)
    ws = torch.zeros(sv.sv_tree_sampling_workspace_bytes(big.B, big.N, big.V, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    for cfg in (big, small, big):
        inp = sample_tree_inputs(cfg, device="cuda")
        out = _call(sv, inp, workspace_tensor=ws)
        assert int(out["err_flags"].item()) == 0
        _compare(out, _oracle(inp), cfg.name)
        assert int(ws.count_nonzero().item()) == 0


def test_split_walk_parity_and_workspace(sv):
    # Few sequences of long rows: each sequence's walk is shared by several
    # workgroups (up to eight, one slice of the runs of every pass each).
    base = SAMPLE_TREE_CONFIGS["c4s"]
    cases = [
        base.with_(name="tree_sampling_split_b3_v128256", B=3, N=30, V=128256, variant=61),
        base.with_(name="tree_sampling_split_b5_v64000", B=5, N=64, V=64000, variant=62),
        base.with_(name="tree_sampling_split_b2_v40000_f32", B=2, N=20, V=40000, dtype="f32", variant=63),
    ]
    star = base.with_(name="tree_sampling_split_star", B=4, N=40, V=128256, variant=64)
    nbytes = max(sv.sv_tree_sampling_workspace_bytes(c.B, c.N, c.V, torch.float32 if c.dtype == "f32"
                                                     else torch.bfloat16) for c in cases + [star])
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for round_ in range(2):
        for cfg in cases:
            _say("split walk round", round_, cfg.name)
            inp = sample_tree_inputs(cfg, device="cuda")
            out = _call(sv, inp, workspace_tensor=ws)
            assert int(out["err_flags"].item()) == 0
            assert int(ws.count_nonzero().item()) == 0, f"workspace dirty after {cfg.name}"
            _compare(out, _oracle(inp), cfg.name)
    # a star of 40 children (many passes at the root), and per-sequence errors
    cfg = star
    inp = sample_tree_inputs(cfg, device="cuda", parents=np.full(cfg.N, -1))
    ref = _oracle(inp)
    _say("split walk star tree")
    out = _call(sv, inp, workspace_tensor=ws)
    assert int(out["err_flags"].item()) == 0
    assert int(ws.count_nonzero().item()) == 0
    _compare(out, ref, cfg.name)
    inp["node_tokens"][1, 3] = -1                 # a token outside [0, V)
    inp["target"][2, 0, 17] = float("nan")        # a non-finite root row
    _say("split walk star tree with error sequences")
    out = _call(sv, inp, workspace_tensor=ws)
    assert int(out["err_flags"].item()) == sv.SV_ERRF_TOKEN | sv.SV_ERRF_NONFINITE
    assert int(ws.count_nonzero().item()) == 0
    acc = _np(out["accept_len"])
    assert acc[1] == -1 and acc[2] == -1
    good = [0, 3]
    _compare({k: v[good] for k, v in out.items() if k != "err_flags"}, {k: v[good] for k, v in ref.items()},
             cfg.name + " (clean sequences)")


def test_split_walks_on_concurrent_streams(sv):
    # Two calls whose split walks together hold more workgroups than the GPU
    # has compute units, launched on two streams at once: every wait must end
    # and both must give the same outputs as when each runs alone.
    base = SAMPLE_TREE_CONFIGS["c4s"]
    cfg_a = base.with_(name="tree_sampling_concurrent_a", B=24, N=30, V=128256, variant=71)
    cfg_b = base.with_(name="tree_sampling_concurrent_b", B=16, N=64, V=100000, variant=72)
    inp_a = sample_tree_inputs(cfg_a, device="cuda")
    inp_b = sample_tree_inputs(cfg_b, device="cuda")
    _say("concurrent split walks: references")
    ref_a = _call(sv, inp_a)
    ref_b = _call(sv, inp_b)
    assert int(ref_a["err_flags"].item()) == 0 and int(ref_b["err_flags"].item()) == 0
    _compare(ref_a, _oracle(inp_a), cfg_a.name)
    _compare(ref_b, _oracle(inp_b), cfg_b.name)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    _say("concurrent split walks: two streams")
    for _ in range(4):
        with torch.cuda.stream(s1):
            oa = sv.sv_verify_tree_sampling(inp_a["target"], inp_a["draft"], inp_a["node_tokens"], inp_a["parents"],
                                            inp_a["temperature"], inp_a["uniforms"], stream=s1)
        with torch.cuda.stream(s2):
            ob = sv.sv_verify_tree_sampling(inp_b["target"], inp_b["draft"], inp_b["node_tokens"], inp_b["parents"],
                                            inp_b["temperature"], inp_b["uniforms"], stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert int(oa["err_flags"].item()) == 0 and int(ob["err_flags"].item()) == 0
        for k in ("accept_len", "path_nodes", "next_token"):
            assert torch.equal(oa[k], ref_a[k]), k
            assert torch.equal(ob[k], ref_b[k]), k


def _chi2_ok(counts, probs, label, level, pvals, min_expected=5.0):
    from scipy import stats
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    c_s, e_s = counts[order], exp[order]
    # pool the categories with small expected counts into one
    small = np.cumsum(e_s) < min_expected * 4
    obs = np.concatenate([[c_s[small].sum()], c_s[~small]]) if small.any() else c_s
    ex = np.concatenate([[e_s[small].sum()], e_s[~small]]) if small.any() else e_s
    keep = ex > 0
    obs, ex = obs[keep], ex[keep]
    ex = ex * obs.sum() / ex.sum()
    p = stats.chisquare(obs, ex).pvalue
    print(f"{label}: n {int(n)}, categories {len(obs)}, chi-square p-value {p:.3g} (bar {level:.3g})", flush=True)
    pvals.append(float(p))
    return p > level


@pytest.mark.slow
def test_monte_carlo_losslessness(sv):
    # one tree and one pair of logit tensors shared by every sequence; the
    # sequences differ in their drafted node tokens and uniforms. Four
    # chi-square tests at an overall level of 0.01 (Bonferroni: each p-value
    # must exceed 0.0025).
    B = 1 << 20
    level = 0.01 / 4
    parents = np.array([-1, -1, -1, 0, 0, 1], dtype=np.int32)
    N, V = len(parents), 64
    cfg = SAMPLE_TREE_CONFIGS["c4s"].with_(name="tree_sampling_mc", B=1, N=N, V=V, dtype="bf16", target_sigma=1.2,
                                           draft_sigma=1.0, temperature=1.0, variant=61)
    one = sample_tree_inputs(cfg, device="cuda", parents=parents)
    target = one["target"].expand(B, N + 1, V).contiguous()
    draft = one["draft"].expand(B, N + 1, V).contiguous()
    T = torch.ones(B, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed_stream(61, 0, 7).integers(0, 2 ** 62)))
    pos_parent = torch.tensor(np.where(parents < 0, 0, parents + 1), dtype=torch.int64, device="cuda")
    tokens = sample_draft_tokens_gumbel(draft[:, pos_parent], T, g)
    uniforms = torch.rand((B, N + 1), generator=g, device="cuda", dtype=torch.float32)
    out = sv.sv_verify_tree_sampling(target, draft, tokens, torch.from_numpy(parents).cuda(), T, uniforms)
    torch.cuda.synchronize()
    assert int(out["err_flags"].item()) == 0
    acc = _np(out["accept_len"]).astype(np.int64)
    path = _np(out["path_nodes"]).astype(np.int64)
    nxt = _np(out["next_token"]).astype(np.int64)
    tok = _np(tokens).astype(np.int64)
    rows = np.arange(B)
    first = np.where(acc >= 1, tok[rows, np.maximum(path[:, 0], 0)], nxt)
    t64 = _np(one["target"][0].double())
    p_root = oracle.temperature_softmax(t64[0], 1.0)
    pvals = []
    assert _chi2_ok(np.bincount(first, minlength=V), p_root, "first emitted token", level, pvals)
    # given that child v of the root was accepted first, the next emitted token follows p at v's position
    for v in (0, 1, 2):
        sel = (acc >= 1) & (path[:, 0] == v)
        nxt_tok = np.where(acc[sel] >= 2, tok[rows[sel], np.maximum(path[sel, 1], 0)], nxt[sel])
        assert _chi2_ok(np.bincount(nxt_tok, minlength=V), oracle.temperature_softmax(t64[v + 1], 1.0),
                        f"token after accepted child {v}", level, pvals)
    record_parity("tree_sampling_mc", call="sv_verify_tree_sampling", trials=B, chi2_pvalues=pvals,
                  bonferroni_bar_each=level)
