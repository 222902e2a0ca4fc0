"""Pins for the oracle's draft-side sampling (``oracle.sample_rows``).

The function is the temperature softmax followed by the inverse CDF over
ascending token id. It is pinned here against facts that do not come from
the function itself:

* the law of the drawn token: 10^6 seeded draws on a 16-token vocabulary match
  the temperature softmax (chi-square), and a planted mistake (the temperature
  dropped from the softmax) fails the same test;
* closed forms: equal logits give token floor(u * V); a logit far above the
  others is always drawn; T and the logits scale together;
* brute force: a pure-Python loop (math.exp, running sums) on tiny rows.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.specverify_oracle as ov
from oracle import FLAG_WINDOW, sample_rows, verify_chain

from test_oracle_mc import _chi2_pvalue


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


def test_marginal_matches_temperature_softmax():
    rng = _rng(7)
    V, n, T = 16, 1_000_000, 0.8
    row = rng.normal(0.0, 2.0, V)
    u = rng.random(n)
    t, prob, _, _ = sample_rows(np.broadcast_to(row, (n, V)), np.full(n, T), u)
    q = np.exp(row / T - (row / T).max())
    q /= q.sum()
    assert _chi2_pvalue(np.bincount(t, minlength=V), q) > 0.01
    np.testing.assert_allclose(prob, q[t], rtol=1e-12)


def test_planted_mistake_fails_the_marginal_test(monkeypatch):
    # an oracle that forgot the temperature must not pass the law test
    rng = _rng(8)
    V, n, T = 16, 1_000_000, 0.5
    row = rng.normal(0.0, 2.0, V)
    u = rng.random(n)
    real = ov.temperature_softmax
    monkeypatch.setattr(ov, "temperature_softmax", lambda logits, temperature: real(logits, np.ones_like(temperature)))
    t, _, _, _ = ov.sample_rows(np.broadcast_to(row, (n, V)), np.full(n, T), u)
    q = np.exp(row / T - (row / T).max())
    q /= q.sum()
    assert _chi2_pvalue(np.bincount(t, minlength=V), q) < 1e-6


def test_equal_logits_give_floor_u_times_v():
    rng = _rng(9)
    for V in (2, 7, 16, 1000):
        u = rng.random(4096)
        frac = u * V - np.floor(u * V)
        keep = (frac > 1e-9) & (frac < 1 - 1e-9)  # away from the boundaries between tokens
        t, prob, _, _ = sample_rows(np.full((keep.sum(), V), 3.25), np.full(keep.sum(), 0.7), u[keep])
        assert np.array_equal(t, np.floor(u[keep] * V).astype(np.int64))
        np.testing.assert_allclose(prob, 1.0 / V, rtol=1e-12)


def test_dominant_logit_is_always_drawn():
    rng = _rng(10)
    R, V = 512, 64
    logits = rng.normal(0.0, 1.0, (R, V))
    hot = rng.integers(0, V, R)
    logits[np.arange(R), hot] = 1000.0
    t, prob, _, _ = sample_rows(logits, np.full(R, 1.3), rng.random(R))
    assert np.array_equal(t, hot)
    np.testing.assert_allclose(prob, 1.0, rtol=1e-12)


def test_temperature_scales_with_the_logits():
    rng = _rng(11)
    R, V = 256, 300
    logits = rng.normal(0.0, 3.0, (R, V))
    T = rng.uniform(0.3, 1.7, R)
    u = rng.random(R)
    a = sample_rows(logits, T, u)
    b = sample_rows(logits / T[:, None], None, u)
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


def _brute(row, T, u):
    e = [math.exp((x - max(row)) / T) for x in row]
    total = 0.0
    for x in e:
        total += x
    run = 0.0
    for i, x in enumerate(e):
        run += x
        if run > u * total:
            return i, x / total
    return max(i for i, x in enumerate(e) if x > 0), e[-1] / total


def test_brute_force_on_tiny_rows():
    rng = _rng(12)
    checked = 0
    for _ in range(2000):
        V = int(rng.integers(1, 7))
        row = list(rng.normal(0.0, 2.0, V))
        T = float(rng.uniform(0.2, 2.0))
        u = float(rng.random())
        t, prob, lo, hi = sample_rows(np.array([row]), np.array([T]), np.array([u]))
        if min(abs(u - lo[0]), abs(hi[0] - u)) < FLAG_WINDOW:
            continue  # a near-boundary draw: either neighbour is a correct answer
        bt, bp = _brute(row, T, u)
        assert t[0] == bt
        assert prob[0] == pytest.approx(bp, rel=1e-12)
        checked += 1
    assert checked > 1900


def test_drawn_token_lies_inside_its_cdf_interval():
    rng = _rng(13)
    R, V = 1000, 50
    t, prob, lo, hi = sample_rows(rng.normal(0, 2, (R, V)), np.full(R, 0.9), u := rng.random(R))
    assert np.all(lo <= u) and np.all(u < hi)
    np.testing.assert_allclose(hi - lo, prob, atol=1e-12)


def test_same_draw_as_the_bonus_of_a_zero_length_chain():
    # with no drafted tokens, verification draws its bonus token from p_0 with
    # the row's uniform: the same operation on the same inputs
    rng = _rng(14)
    R, V = 64, 500
    logits = rng.normal(0, 2, (R, V))
    T = rng.uniform(0.5, 1.5, R)
    u = rng.random(R)
    t, _, _, _ = sample_rows(logits, T, u)
    r = verify_chain(logits[:, None, :], np.zeros((R, 0, V)), np.zeros((R, 0), np.int64), T, u[:, None])
    assert np.array_equal(r["out_tokens"][:, 0], t)
