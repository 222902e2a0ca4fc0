"""Pins for the greedy tree-verification and tree-mask oracles.

* Greedy tree acceptance vs brute force over explicit root-to-leaf paths, for
  every parent array with up to 6 nodes, random tokens over a 3-4 token
  vocabulary, integer logits (so argmax ties happen).
* A chain-shaped tree reduces to greedy chain matching; a star-shaped tree
  accepts at most one node.
* The mask vs Warshall's transitive closure of the parent relation; chain =>
  lower-triangular ones, star => identity.
* The pages' own trees: the EAGLE-2 figure, the SpecInfer top-2 tree and the
  sequence diagram's four proposals.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import node_depths, tree_mask, verify_tree_greedy


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


def _all_parent_arrays(n):
    return itertools.product(*[range(-1, i) for i in range(n)])


def _first_max(row):
    best = 0
    for v in range(1, len(row)):
        if row[v] > row[best]:
            best = v
    return best


def _brute_force(logits, tokens, parents):
    """Enumerate root-to-leaf paths; keep the longest accepted prefix."""
    N = len(parents)
    children = {i: [c for c in range(N) if parents[c] == i] for i in range(-1, N)}
    paths = []

    def walk(node, prefix):
        kids = children[node]
        if not kids and prefix:
            paths.append(prefix)
        for c in kids:
            walk(c, prefix + [c])

    walk(-1, [])
    best_len, best_end = 0, None
    for path in paths:
        n_ok = 0
        prev_pos = 0
        for node in path:
            if tokens[node] != _first_max(logits[prev_pos]):
                break
            n_ok += 1
            prev_pos = node + 1
        if n_ok == 0:
            continue
        end = path[n_ok - 1]
        if n_ok > best_len or (n_ok == best_len and end < best_end):
            best_len, best_end = n_ok, end
    if best_end is None:
        return 0, None, _first_max(logits[0]), None
    return best_len, None, _first_max(logits[best_end + 1]), best_end


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_greedy_tree_matches_brute_force_exhaustively(n):
    rng = _rng(200 + n)
    for parents in _all_parent_arrays(n):
        parents = np.array(parents)
        V = int(rng.integers(3, 5))
        B = 3
        logits = rng.integers(0, 3, (B, n + 1, V)).astype(np.float64)  # small ints: ties
        tokens = rng.integers(0, V, (B, n))
        # make acceptance likely: copy the argmax into some node tokens
        for b in range(B):
            for i in range(n):
                if rng.random() < 0.6:
                    pos = 0 if parents[i] < 0 else parents[i] + 1
                    tokens[b, i] = _first_max(logits[b, pos])
        r = verify_tree_greedy(logits, tokens, parents)
        for b in range(B):
            bf = _brute_force(logits[b], tokens[b], parents)
            assert r["accept_len"][b] == bf[0]
            assert r["next_token"][b] == bf[2]
            if bf[0] > 0:
                end = bf[3]
                chain = []
                k = end
                while k >= 0:
                    chain.append(k)
                    k = parents[k]
                assert r["path_nodes"][b, : bf[0]].tolist() == chain[::-1]
            assert np.all(r["path_nodes"][b, bf[0]:] == -1)


def test_argmax_ties_take_lowest_id():
    logits = np.array([[[1.0, 5.0, 5.0, 2.0], [0.0, 0.0, 0.0, 0.0]]])
    r = verify_tree_greedy(logits, np.array([[2]]), np.array([-1]))
    assert r["argmax"][0, 0] == 1 and r["argmax"][0, 1] == 0
    assert r["accept_len"][0] == 0 and r["next_token"][0] == 1
    r = verify_tree_greedy(logits, np.array([[1]]), np.array([-1]))
    assert r["accept_len"][0] == 1 and r["next_token"][0] == 0


def test_chain_tree_is_greedy_chain_matching():
    rng = _rng(210)
    N, V = 7, 5
    parents = np.arange(-1, N - 1)
    for _ in range(50):
        logits = rng.normal(0, 1, (1, N + 1, V))
        g = logits[0].argmax(axis=-1)
        tokens = g[:N].copy()
        cut = int(rng.integers(0, N + 1))
        if cut < N:
            tokens[cut] = (g[cut] + 1) % V
        r = verify_tree_greedy(logits, tokens[None], parents)
        assert r["accept_len"][0] == cut
        assert r["next_token"][0] == g[cut]
        assert r["path_nodes"][0, :cut].tolist() == list(range(cut))


def test_star_tree_accepts_at_most_one():
    rng = _rng(211)
    N, V = 6, 3
    parents = np.full(N, -1)
    for _ in range(50):
        logits = rng.normal(0, 1, (1, N + 1, V))
        tokens = rng.integers(0, V, (1, N))
        r = verify_tree_greedy(logits, tokens, parents)
        g0 = logits[0, 0].argmax()
        match = np.flatnonzero(tokens[0] == g0)
        if len(match):
            assert r["accept_len"][0] == 1 and r["path_nodes"][0, 0] == match[0]
            assert r["next_token"][0] == logits[0, match[0] + 1].argmax()
        else:
            assert r["accept_len"][0] == 0 and r["next_token"][0] == g0


def test_invalid_tree_rows():
    logits = np.zeros((2, 3, 4))
    r = verify_tree_greedy(logits, np.array([[0, 1], [0, 7]]), np.array([-1, 0]))
    assert r["accept_len"][0] >= 0 and r["accept_len"][1] == -1
    r = verify_tree_greedy(logits, np.array([[0, 1], [0, 1]]), np.array([-1, 1]))
    assert np.all(r["accept_len"] == -1)


# ----------------------------------------------------------------------------- mask

def _warshall(parents):
    N = len(parents)
    reach = np.zeros((N, N), dtype=bool)
    for i, par in enumerate(parents):
        if par >= 0:
            reach[i, par] = True
    for k in range(N):
        reach |= reach[:, k:k + 1] & reach[k:k + 1, :]
    return (reach | np.eye(N, dtype=bool)).astype(np.uint8)


def test_mask_matches_transitive_closure():
    rng = _rng(220)
    for N in (1, 2, 5, 17, 64, 100):
        for _ in range(5):
            parents = np.array([-1 if i == 0 or rng.random() < 0.2 else int(rng.integers(0, i)) for i in range(N)])
            np.testing.assert_array_equal(tree_mask(parents), _warshall(parents))


def test_mask_chain_and_star():
    N = 9
    np.testing.assert_array_equal(tree_mask(np.arange(-1, N - 1)), np.tril(np.ones((N, N), np.uint8)))
    np.testing.assert_array_equal(tree_mask(np.full(N, -1)), np.eye(N, dtype=np.uint8))


def test_mask_rejects_bad_parents():
    with pytest.raises(ValueError):
        tree_mask(np.array([-1, 1]))
    with pytest.raises(ValueError):
        tree_mask(np.array([0]))
    with pytest.raises(ValueError):
        tree_mask(np.array([-1, -2]))


def test_depths():
    np.testing.assert_array_equal(node_depths(np.array([-1, 0, 1, -1, 3, 0])), [1, 2, 3, 1, 2, 2])


# ----------------------------------------------------------------------------- the pages' trees

def test_eagle2_figure_tree(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "eagle2_tree_figure.json")))
    names = g["nodes"]
    idx = {n: i for i, n in enumerate(names)}
    parents = np.array([-1 if g["edges_parent_of"][n] == g["root"] else idx[g["edges_parent_of"][n]]
                        for n in names])
    m = tree_mask(parents)
    for n in names:
        row = {names[j] for j in np.flatnonzero(m[idx[n]])}
        expect = {n}
        p = g["edges_parent_of"][n]
        while p != g["root"]:
            expect.add(p)
            p = g["edges_parent_of"][p]
        assert row == expect
    # Node 1 ("Computing") and its children are verified together; a target
    # whose argmax follows Computing -> Algorithms accepts that 2-node path.
    V = len(names) + 1
    vocab = {n: i for i, n in enumerate(names)}
    logits = np.zeros((1, len(names) + 1, V))
    logits[0, 0, vocab["Computing"]] = 5.0
    logits[0, idx["Computing"] + 1, vocab["Algorithms"]] = 5.0
    logits[0, idx["Algorithms"] + 1, V - 1] = 5.0
    tokens = np.array([[vocab[n] for n in names]])
    r = verify_tree_greedy(logits, tokens, parents)
    assert r["accept_len"][0] == 2
    assert [names[i] for i in r["path_nodes"][0, :2]] == ["Computing", "Algorithms"]
    assert r["next_token"][0] == V - 1


def test_specinfer_top2_tree(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "specinfer_top2_tree.json")))
    w1, w2 = g["levels"]
    parents = np.array([-1] * w1 + [i // w2 for i in range(w1 * w2)])
    m = tree_mask(parents)
    assert m.shape == (w1 + w1 * w2,) * 2
    assert m.sum() == w1 + 2 * w1 * w2  # level-1 rows: self; level-2 rows: self + parent
    assert np.all(node_depths(parents) == np.array([1] * w1 + [2] * (w1 * w2)))


def test_sequence_diagram_greedy_chain(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "sequence_diagram_greedy.json")))
    K = len(g["proposals"])
    V = 10
    rng = _rng(230)
    logits = rng.normal(0, 1, (1, K + 1, V))
    argmax = logits[0].argmax(axis=-1)
    tokens = np.array([[argmax[k] if g["matching"][k] else (argmax[k] + 1) % V for k in range(K)]])
    r = verify_tree_greedy(logits, tokens, np.arange(-1, K - 1))
    n_acc = len(g["accepted"])
    assert r["accept_len"][0] == n_acc
    assert r["next_token"][0] == argmax[n_acc]  # the target's own token after the accepted prefix
    assert int(r["accept_len"][0]) + g["extra_tokens_from_target"] == 4
