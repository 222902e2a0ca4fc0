"""The seeded input generators: determinism, shapes, dtypes, value ranges, tree shape."""
import numpy as np
import pytest
import torch
from scipy import stats

from workloads import (
    CHAIN_CONFIGS,
    MC_CONFIG,
    TREE_CONFIGS,
    chain_inputs,
    mc_chain_inputs,
    tree_inputs,
    tree_parents_ranked,
)
from workloads.synth import chain_uniforms


def test_chain_inputs_deterministic_and_shaped():
    cfg = CHAIN_CONFIGS["c1"].with_(B=3, V=1000)
    a = chain_inputs(cfg)
    b = chain_inputs(cfg)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert a["target"].shape == (3, 5, 1000) and a["target"].dtype == torch.float32
    assert a["draft"].shape == (3, 4, 1000)
    assert a["draft_tokens"].dtype == torch.int32 and a["draft_tokens"].shape == (3, 4)
    assert a["uniforms"].shape == (3, 5) and a["uniforms"].dtype == torch.float32
    assert float(a["uniforms"].min()) >= 0.0 and float(a["uniforms"].max()) < 1.0
    assert int(a["draft_tokens"].min()) >= 0 and int(a["draft_tokens"].max()) < 1000


def test_bf16_config_rounds_independently():
    cfg = CHAIN_CONFIGS["c2"].with_(B=2, V=4096)
    x = chain_inputs(cfg)
    assert x["target"].dtype == torch.bfloat16 and x["draft"].dtype == torch.bfloat16
    assert torch.all(x["temperature"] == np.float32(0.7))
    # the Zipf log-prior lowers late ids on average
    t = x["target"].float()
    assert float(t[..., :100].mean()) > float(t[..., -100:].mean()) + 5.0


def test_per_row_temperature_range():
    cfg = CHAIN_CONFIGS["c3_s1.0"].with_(B=64, V=512)
    T = chain_inputs(cfg)["temperature"]
    assert float(T.min()) >= 0.3 and float(T.max()) <= 1.3 and len(set(T.tolist())) > 50


def test_uniform_iterations_differ():
    cfg = CHAIN_CONFIGS["c5"].with_(B=4)
    assert not torch.equal(chain_uniforms(cfg, 0), chain_uniforms(cfg, 1))


def test_draft_tokens_follow_draft_distribution():
    # Gumbel-max on the stored draft logits draws x ~ softmax(d / T).
    x = mc_chain_inputs(MC_CONFIG, 200_000)
    d = x["draft_row"].double().numpy()
    T = float(x["temperature"][0])
    for k in range(d.shape[0]):
        a = d[k] / T
        q = np.exp(a - a.max())
        q /= q.sum()
        n = len(x["draft_tokens"])
        counts = np.bincount(x["draft_tokens"][:, k].numpy(), minlength=d.shape[1])
        big = q * n >= 5
        obs = counts[big].astype(float)
        exp = q[big] * n
        if (~big).any():
            obs = np.append(obs, counts[~big].sum())
            exp = np.append(exp, q[~big].sum() * n)
        assert stats.chisquare(obs, exp * obs.sum() / exp.sum()).pvalue > 1e-4


def test_tree_parents_shape():
    parents, ranks = tree_parents_ranked((4, 3, 2, 2, 1), 64)
    assert len(parents) == 64
    assert all(p == -1 or 0 <= p < i for i, p in enumerate(parents))
    depth = np.zeros(64, int)
    for i, p in enumerate(parents):
        depth[i] = 1 if p < 0 else depth[p] + 1
    assert np.bincount(depth)[1:].tolist() == [4, 9, 15, 23, 13]
    # sibling ranks are 0..n-1 under every parent
    for par in set(parents.tolist()):
        rk = sorted(ranks[parents == par].tolist())
        assert rk == list(range(len(rk)))
    with pytest.raises(ValueError):
        tree_parents_ranked((2, 2), 7)


def test_tree_inputs_small():
    cfg = TREE_CONFIGS["c4"].with_(B=3, V=300)
    x = tree_inputs(cfg)
    y = tree_inputs(cfg)
    assert torch.equal(x["node_tokens"], y["node_tokens"])
    assert x["target"].shape == (3, 65, 300) and x["target"].dtype == torch.bfloat16
    assert x["node_tokens"].shape == (3, 64)
    parents = x["parents"].numpy()
    # most first-rank nodes carry the parent position's top token
    t = x["target"].float().numpy()
    _, ranks = tree_parents_ranked(cfg.branching, cfg.N)
    hits = total = 0
    for b in range(3):
        for i in range(64):
            if ranks[i] == 0:
                pos = 0 if parents[i] < 0 else parents[i] + 1
                total += 1
                hits += int(x["node_tokens"][b, i]) == int(np.argmax(t[b, pos]))
    assert hits / total > 0.5
