"""Pins of the oracle's per-position entropy (CPU only).

The entropy of a temperature softmax is pinned by closed forms (uniform rows,
two-token rows through the logistic function), by the Gibbs identity
H = logsumexp(a) - E_p[a] for a = logits / T (scipy's logsumexp), by its limits
and bounds, and by its monotone growth with the temperature.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import entropy, temperature_softmax, verify_chain

RNG = lambda seed: np.random.Generator(np.random.Philox(seed))  # noqa: E731


@pytest.mark.parametrize("V", [1, 2, 7, 32000])
def test_uniform_rows_give_log_v(V):
    p = temperature_softmax(np.full((3, V), 1.7), np.array([0.4, 1.0, 3.0]))
    assert np.allclose(entropy(p), math.log(V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("delta,T", [(0.0, 1.0), (1.3, 0.7), (-4.0, 1.0), (9.0, 2.5)])
def test_two_tokens_is_the_binary_entropy(delta, T):
    # p(token 1) is the logistic function of (l1 - l0) / T
    s = 1.0 / (1.0 + math.exp(-delta / T))
    h = -(s * math.log(s) + (1.0 - s) * math.log(1.0 - s))
    p = temperature_softmax(np.array([[0.25, 0.25 + delta]]), np.array([T]))
    assert abs(entropy(p)[0] - h) < 1e-14


def test_gibbs_identity():
    # H(softmax(a)) = logsumexp(a) - sum_v p(v) a_v
    rng = RNG(3)
    logits = rng.normal(0, 3, (6, 5000))
    T = rng.uniform(0.3, 1.5, 6)
    a = logits / T[:, None]
    p = temperature_softmax(logits, T)
    expect = logsumexp(a, axis=1) - (p * a).sum(axis=1)
    assert np.allclose(entropy(p), expect, rtol=1e-12, atol=1e-12)


def test_bounds_and_limits():
    rng = RNG(4)
    logits = rng.normal(0, 2, (8, 1000))
    h = entropy(temperature_softmax(logits, np.ones(8)))
    assert np.all(h >= 0) and np.all(h <= math.log(1000))
    # T -> 0 with a unique maximum: a point mass, entropy 0
    logits[:, 17] = logits.max(axis=1) + 1.0
    assert np.all(entropy(temperature_softmax(logits, np.full(8, 1e-3))) < 1e-200)
    # T -> inf: uniform
    assert np.allclose(entropy(temperature_softmax(logits, np.full(8, 1e9))), math.log(1000), atol=1e-6)


def test_grows_with_temperature():
    # dH/dT = Var_p(a) / T >= 0 for a softmax at temperature T
    rng = RNG(5)
    logits = rng.normal(0, 3, (4, 2000))
    Ts = [0.2, 0.5, 0.9, 1.4, 3.0]
    h = np.stack([entropy(temperature_softmax(logits, np.full(4, T))) for T in Ts])
    assert np.all(np.diff(h, axis=0) > 0)


def test_zero_probability_tokens_do_not_count():
    rng = RNG(6)
    row = rng.normal(0, 2, 300)
    masked = row.copy()
    masked[::3] = -np.inf
    p_masked = temperature_softmax(masked[None], np.array([0.8]))
    p_kept = temperature_softmax(np.delete(row, np.s_[::3])[None], np.array([0.8]))
    assert abs(entropy(p_masked)[0] - entropy(p_kept)[0]) < 1e-12


def test_chain_reports_the_entropy_of_every_position():
    rng = RNG(7)
    B, K, V = 3, 4, 500
    t = rng.normal(0, 3, (B, K + 1, V))
    d = t[:, :K] + rng.normal(0, 1, (B, K, V))
    T = np.array([0.7, 1.0, 1.3])
    x = rng.integers(0, V, (B, K))
    out = verify_chain(t, d, x, T, rng.random((B, K + 1)), with_entropy=True)
    for b in range(B):
        a_t = t[b] / T[b]
        a_d = d[b] / T[b]
        ref_t = [logsumexp(r) - (np.exp(r - logsumexp(r)) * r).sum() for r in a_t]
        ref_d = [logsumexp(r) - (np.exp(r - logsumexp(r)) * r).sum() for r in a_d]
        assert np.allclose(out["entropy"][b], ref_t + ref_d, rtol=1e-12, atol=1e-12)
