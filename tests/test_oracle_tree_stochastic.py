"""Pins of the oracle's sampling (stochastic) tree verification (CPU only).

* A chain-shaped tree is chain verification: identical outputs to
  verify_chain on the same logits and uniforms.
* Losslessness: with children drawn i.i.d. from the draft distribution at
  their parent, the token emitted at each depth follows the target's
  distribution at that depth (chi-square, seeded Monte Carlo), and two
  mistakes planted in the oracle (no residual update between siblings; the
  ratio q/p in place of p/q) fail the same test.
* The rule itself, by exact enumeration on star trees: the distribution of the
  emitted token is p.
* Edge cases: draft = target accepts the first child at every node; invalid
  rows are reported.
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.specverify_oracle as so

RNG = lambda seed: np.random.Generator(np.random.Philox(seed))  # noqa: E731


def _softmax(a):
    e = np.exp(a - a.max())
    return e / e.sum()


@pytest.mark.parametrize("B,K,V,seed", [(6, 4, 50, 1), (5, 1, 7, 2), (4, 6, 300, 3)])
def test_chain_tree_is_chain_verification(B, K, V, seed):
    rng = RNG(seed)
    t = rng.normal(0, 2, (B, K + 1, V))
    dr = t[:, :K] + rng.normal(0, 1, (B, K, V))
    T = rng.uniform(0.5, 1.5, B)
    x = np.stack([[rng.choice(V, p=_softmax(dr[b, k] / T[b])) for k in range(K)] for b in range(B)])
    u = rng.random((B, K + 1))
    ch = oracle.verify_chain(t, dr, x, T, u)
    parents = np.arange(-1, K - 1)
    # the draft row at node k's position (k + 1) is unused by a chain tree's
    # last node only if it is a leaf; rows 0..K-1 are the chain's draft rows
    d_full = np.concatenate([dr, rng.normal(0, 1, (B, 1, V))], axis=1)
    tr = oracle.verify_tree_stochastic(t, d_full, x, parents, T, u)
    assert np.array_equal(tr["accept_len"], ch["accept_len"])
    for b in range(B):
        j = ch["accept_len"][b]
        assert np.array_equal(tr["emitted"][b, :j + 1], ch["out_tokens"][b, :j + 1])
        assert tr["next_token"][b] == ch["out_tokens"][b, j]
        assert list(tr["path_nodes"][b, :j]) == list(range(j))


MC_TRIALS = 120_000


def _mc_tree(trials, seed, V=5):
    """Root with 3 children, each with 2 children; the target and draft logits
    depend on the depth only; children drawn i.i.d. from q at their parent."""
    rng = RNG(seed)
    lt = rng.normal(0, 1.5, (3, V))
    ld = lt + rng.normal(0, 1.2, (3, V))
    parents = np.array([-1, -1, -1, 0, 0, 1, 1, 2, 2])
    depth = np.array([1, 1, 1, 2, 2, 2, 2, 2, 2])
    N = len(parents)
    q = [_softmax(ld[k]) for k in range(3)]
    tok = np.empty((trials, N), dtype=np.int64)
    for i in range(N):
        tok[:, i] = rng.choice(V, size=trials, p=q[depth[i] - 1])
    pos_depth = np.concatenate([[0], depth])  # depth of the distribution at each position
    t = np.broadcast_to(lt[pos_depth], (trials, N + 1, V))
    d = np.broadcast_to(ld[pos_depth], (trials, N + 1, V))
    u = rng.random((trials, N + 1))
    p = [_softmax(lt[k]) for k in range(3)]
    return t, d, tok, parents, np.ones(trials), u, p


def _depth_pvalues(out, p, V):
    em, alen = out["emitted"], out["accept_len"]
    pv = []
    for k in range(3):
        reached = alen >= k
        counts = np.bincount(em[reached, k], minlength=V)
        pv.append(stats.chisquare(counts, p[k] * reached.sum()).pvalue)
    return pv


def test_emitted_tokens_follow_the_target_at_every_depth():
    V = 5
    t, d, tok, parents, T, u, p = _mc_tree(MC_TRIALS, seed=11, V=V)
    out = oracle.verify_tree_stochastic(t, d, tok, parents, T, u)
    assert np.all(out["valid"])
    pv = _depth_pvalues(out, p, V)
    assert min(pv) > 0.01, pv
    # all three depths are reached often enough to matter
    assert (out["accept_len"] >= 2).mean() > 0.1


@pytest.mark.parametrize("mistake", ["no_residual_update", "inverted_ratio"])
def test_planted_mistakes_fail_the_same_test(monkeypatch, mistake):
    V = 5
    if mistake == "no_residual_update":
        monkeypatch.setattr(so, "residual_weights", lambda P, q: np.asarray(P, np.float64))
    else:
        monkeypatch.setattr(so, "acceptance_probability", lambda px, qx: np.minimum(1.0, qx / px))
    t, d, tok, parents, T, u, p = _mc_tree(MC_TRIALS, seed=11, V=V)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = so.verify_tree_stochastic(t, d, tok, parents, T, u)
    pv = min(_depth_pvalues(out, p, V))
    print(mistake, "smallest p-value", pv)
    assert pv < 1e-6


@pytest.mark.parametrize("V,m,seed", [(4, 2, 21), (3, 3, 22), (5, 2, 23)])
def test_rule_is_lossless_by_enumeration(V, m, seed):
    # star tree with m children drawn i.i.d. from q: the emitted token's exact
    # distribution, summed over every children assignment and integrated over
    # the uniforms, equals p
    rng = RNG(seed)
    p = _softmax(rng.normal(0, 1.5, V))
    q = _softmax(rng.normal(0, 1.5, V))
    out = np.zeros(V)
    for xs in itertools.product(range(V), repeat=m):
        w = np.prod(q[list(xs)])
        P, alive = p.copy(), 1.0
        for x in xs:
            a = min(1.0, P[x] / q[x]) if q[x] > 0 else 1.0
            out[x] += w * alive * a
            alive *= 1.0 - a
            r = np.maximum(0.0, P - q)
            if r.sum() > 0:
                P = r / r.sum()
        out += w * alive * P
    assert np.allclose(out, p, rtol=0, atol=1e-12)


def test_identical_draft_accepts_the_first_child_everywhere():
    rng = RNG(31)
    B, V = 4, 40
    parents = np.array([-1, -1, 0, 0, 2, -1])
    N = len(parents)
    t = rng.normal(0, 2, (B, N + 1, V))
    tok = rng.integers(0, V, (B, N))
    out = oracle.verify_tree_stochastic(t, t.copy(), tok, parents, np.ones(B), rng.random((B, N + 1)))
    # first children: 0 -> 2 -> 4 (a leaf)
    assert np.all(out["accept_len"] == 3)
    assert np.all(out["path_nodes"][:, :3] == [0, 2, 4])


def test_invalid_rows_are_reported():
    rng = RNG(32)
    B, V = 3, 10
    parents = np.array([-1, 0])
    t = rng.normal(0, 1, (B, 3, V))
    tok = np.array([[1, 2], [1, V], [0, 0]])
    T = np.array([1.0, 1.0, 0.0])
    out = oracle.verify_tree_stochastic(t, t, tok, parents, T, rng.random((B, 3)))
    assert list(out["valid"]) == [True, False, False]
    assert list(out["accept_len"][1:]) == [-1, -1]
    bad = oracle.verify_tree_stochastic(t, t, tok, np.array([-1, 1]), T, rng.random((B, 3)))
    assert np.all(bad["accept_len"] == -1)
