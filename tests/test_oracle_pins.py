"""Pins for the chain-verification oracle: closed forms, identities, special cases.

Each test fixes the oracle against something other than itself: a textbook
formula, a library routine, an identity the pages state, or a case whose
outcome the pages' rules decide for every uniform.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (
    acceptance_probability,
    inverse_cdf,
    residual_weights,
    temperature_softmax,
    verify_chain,
)


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


# ----------------------------------------------------------------------------- softmax

@pytest.mark.parametrize("T", [0.05, 0.3, 0.7, 1.0, 2.5, 5.0])
def test_softmax_two_tokens_is_logistic(T):
    # Two tokens: p(1) = 1 / (1 + exp(-(l1 - l0) / T)), the logistic function.
    rng = _rng(1)
    l = rng.normal(0.0, 3.0, size=(50, 2))
    p = temperature_softmax(l, np.full(50, T))
    expect = 1.0 / (1.0 + np.exp(-(l[:, 1] - l[:, 0]) / T))
    np.testing.assert_allclose(p[:, 1], expect, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-15)


def test_softmax_uniform_logits_give_uniform_distribution():
    for V in (1, 2, 7, 16, 32000):
        p = temperature_softmax(np.full((1, V), 1.234), np.array([0.7]))
        assert np.all(p == 1.0 / V) or np.allclose(p, 1.0 / V, rtol=1e-15, atol=0)


def test_softmax_temperature_limit_is_argmax():
    # T -> 0: all the mass on the largest logit.
    l = np.array([[0.0, 1.0, 3.0, 2.9]])
    p = temperature_softmax(l, np.array([0.001]))
    assert p[0, 2] == pytest.approx(1.0, abs=1e-15) and p[0, :2].max() < 1e-300
    assert p[0, 3] == pytest.approx(math.exp(-100.0), rel=1e-10)  # exp(-(3.0 - 2.9) / 0.001)


def test_softmax_matches_exp_ratio_for_three_tokens():
    # p_i = 1 / sum_j exp((l_j - l_i)/T), evaluated independently term by term.
    l = np.array([[0.5, -1.25, 2.0]])
    T = 0.8
    p = temperature_softmax(l, np.array([T]))[0]
    for i in range(3):
        expect = 1.0 / sum(math.exp((l[0, j] - l[0, i]) / T) for j in range(3))
        assert p[i] == pytest.approx(expect, rel=1e-14)


# ----------------------------------------------------------------------------- acceptance

def test_acceptance_probability_cases():
    p = np.array([0.3, 0.2, 0.2, 0.0, 0.0, 0.4])
    q = np.array([0.1, 0.2, 0.5, 0.3, 0.0, 0.0])
    a = acceptance_probability(p, q)
    # p >= q: always kept; p < q: kept with probability p/q (pages' rule);
    # p = 0: never; q = 0 < p: always (edge readings).
    np.testing.assert_array_equal(a, [1.0, 1.0, 0.4, 0.0, 0.0, 1.0])


def test_acceptance_rate_is_expected_min():
    # The acceptance rate for x ~ q is E_q[min(1, p/q)] = sum_x min(p(x), q(x)).
    rng = _rng(2)
    for _ in range(20):
        V = int(rng.integers(2, 40))
        p = temperature_softmax(rng.normal(0, 2, (1, V)), np.array([1.0]))[0]
        q = temperature_softmax(rng.normal(0, 2, (1, V)), np.array([1.0]))[0]
        rate = float(np.sum(q * acceptance_probability(p, q)))
        assert rate == pytest.approx(float(np.minimum(p, q).sum()), rel=1e-13)
        # and equals 1 - total variation distance
        assert rate == pytest.approx(1.0 - 0.5 * float(np.abs(p - q).sum()), rel=1e-12)


# ----------------------------------------------------------------------------- residual

def test_residual_mass_is_total_variation():
    rng = _rng(3)
    for _ in range(20):
        V = int(rng.integers(2, 200))
        p = temperature_softmax(rng.normal(0, 3, (1, V)), np.array([1.0]))[0]
        q = temperature_softmax(rng.normal(0, 3, (1, V)), np.array([1.0]))[0]
        r = residual_weights(p, q)
        assert r.sum() == pytest.approx(1.0 - np.minimum(p, q).sum(), abs=1e-14)
        assert r.sum() == pytest.approx(0.5 * np.abs(p - q).sum(), abs=1e-14)
        assert np.all(r[p <= q] == 0.0)
        assert np.all(r[p > q] > 0.0)
        assert (r / r.sum()).sum() == pytest.approx(1.0, abs=1e-14)


def test_residual_completes_the_target_distribution():
    # For x ~ q: P(emit v) = q(v) min(1, p/q) + (1 - sum min(p,q)) * r(v)/S = p(v),
    # the identity behind losslessness, evaluated exactly for random pairs.
    rng = _rng(4)
    for _ in range(20):
        V = int(rng.integers(2, 50))
        p = temperature_softmax(rng.normal(0, 2, (1, V)), np.array([0.9]))[0]
        q = temperature_softmax(rng.normal(0, 2, (1, V)), np.array([0.9]))[0]
        r = residual_weights(p, q)
        emit = q * acceptance_probability(p, q) + (1.0 - np.minimum(p, q).sum()) * r / r.sum()
        np.testing.assert_allclose(emit, p, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- inverse CDF

def test_inverse_cdf_matches_searchsorted():
    rng = _rng(5)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        u = float(rng.random())
        t, lo, hi = inverse_cdf(w[None], np.array([u]))
        c = np.cumsum(w)
        assert int(t[0]) == int(np.searchsorted(c, u * c[-1], side="right"))
        assert w[int(t[0])] > 0
        assert lo[0] <= u < hi[0]


def test_inverse_cdf_boundary_convention():
    # Reading: the first t with cumsum > u * total (strict), ascending ids.
    t, _, _ = inverse_cdf(np.array([[0.5, 0.5]]), np.array([0.5]))
    assert t[0] == 1
    t, _, _ = inverse_cdf(np.array([[0.25, 0.0, 0.75]]), np.array([0.25]))
    assert t[0] == 2  # zero-weight id 1 is never drawn
    t, _, _ = inverse_cdf(np.array([[0.25, 0.0, 0.75]]), np.array([0.0]))
    assert t[0] == 0
    t, _, _ = inverse_cdf(np.array([[0.0, 0.3, 0.0]]), np.array([0.999999]))
    assert t[0] == 1


# ----------------------------------------------------------------------------- chain verification

def _random_case(rng, B, K, V, sigma_t=3.0, sigma_d=1.0, T=None):
    t = rng.normal(0, sigma_t, (B, K + 1, V))
    d = t[:, :K] + rng.normal(0, sigma_d, (B, K, V))
    Tm = np.full(B, 1.0) if T is None else np.asarray(T, float)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1))
    return t, d, x, Tm, u


def test_tokens_per_iteration_in_range():
    rng = _rng(6)
    for K in (0, 1, 3, 8):
        t, d, x, T, u = _random_case(rng, 64, K, 50, T=rng.uniform(0.3, 1.3, 64))
        r = verify_chain(t, d, x, T, u)
        j = r["accept_len"]
        assert np.all((j >= 0) & (j <= K))
        emitted = (r["out_tokens"] >= 0).sum(axis=1)
        np.testing.assert_array_equal(emitted, j + 1)  # between 1 and K+1 tokens
        for b in range(64):
            np.testing.assert_array_equal(r["out_tokens"][b, : j[b]], x[b, : j[b]])


def test_p_ge_q_always_accepted():
    # Draft tokens chosen where p(x) >= q(x): accepted for every u in [0, 1).
    rng = _rng(7)
    B, K, V = 32, 5, 40
    t, d, _, T, _ = _random_case(rng, B, K, V)
    p = temperature_softmax(t, T[:, None])
    q = temperature_softmax(d, T[:, None])
    x = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for k in range(K):
            x[b, k] = int(np.flatnonzero(p[b, k] >= q[b, k])[0])
    for u_val in (0.0, 0.5, np.float32(1.0) - np.float32(2.0 ** -24)):
        u = np.full((B, K + 1), float(u_val))
        r = verify_chain(t, d, x, T, u)
        assert np.all(r["accept_len"] == K)


def test_identical_draft_accepts_everything_and_draws_bonus_from_p():
    rng = _rng(8)
    B, K, V = 40, 4, 64
    t, _, x, T, u = _random_case(rng, B, K, V, T=rng.uniform(0.3, 1.3, 40))
    r = verify_chain(t, t[:, :K].copy(), x, T, u)
    assert np.all(r["accept_len"] == K)
    assert np.all(r["residual_mass"] == -1.0)
    pK = temperature_softmax(t[:, K], T)
    for b in range(B):
        c = np.cumsum(pK[b])
        assert r["out_tokens"][b, K] == np.searchsorted(c, u[b, K] * c[-1], side="right")


def test_disjoint_supports_reject_first_and_draw_from_p():
    # Target mass only on even ids, draft mass only on odd ids (the other
    # logits are so low that exp underflows to exactly 0 in float64).
    rng = _rng(9)
    B, K, V = 30, 3, 20
    t = np.full((B, K + 1, V), -2000.0)
    d = np.full((B, K, V), -2000.0)
    t[:, :, 0::2] = rng.normal(0, 1, (B, K + 1, V // 2))
    d[:, :, 1::2] = rng.normal(0, 1, (B, K, V // 2))
    x = 2 * rng.integers(0, V // 2, (B, K)) + 1
    u = rng.random((B, K + 1))
    T = np.ones(B)
    r = verify_chain(t, d, x, T, u)
    assert np.all(r["accept_len"] == 0)
    np.testing.assert_allclose(r["residual_mass"], 1.0, rtol=1e-14)
    p0 = temperature_softmax(t[:, 0], T)
    for b in range(B):
        c = np.cumsum(p0[b])
        assert r["out_tokens"][b, 0] == np.searchsorted(c, u[b, K] * c[-1], side="right")
        assert r["out_tokens"][b, 0] % 2 == 0


def test_rejection_draws_from_the_residual():
    rng = _rng(10)
    B, K, V = 200, 3, 30
    t, d, x, T, u = _random_case(rng, B, K, V, sigma_d=2.0)
    r = verify_chain(t, d, x, T, u)
    p = temperature_softmax(t, T[:, None])
    q = temperature_softmax(d, T[:, None])
    n_rej = 0
    for b in range(B):
        j = r["accept_len"][b]
        if j == K:
            continue
        n_rej += 1
        w = np.maximum(0.0, p[b, j] - q[b, j])
        c = np.cumsum(w)
        assert r["out_tokens"][b, j] == np.searchsorted(c, u[b, K] * c[-1], side="right")
        assert r["residual_mass"][b] == pytest.approx(1 - np.minimum(p[b, j], q[b, j]).sum(), abs=1e-13)
        assert p[b, j, r["out_tokens"][b, j]] > q[b, j, r["out_tokens"][b, j]]
        # the rejected token's accept test failed, the earlier ones passed
        a = acceptance_probability(p[b, np.arange(K), x[b]], q[b, np.arange(K), x[b]])
        assert np.all(u[b, :j] < a[:j]) and u[b, j] >= a[j]
    assert n_rej > 50


def test_invalid_rows_are_reported():
    rng = _rng(11)
    t, d, x, T, u = _random_case(rng, 6, 3, 10)
    x[1, 2] = 10      # token out of range
    x[2, 0] = -1
    T[3] = 0.0        # non-positive temperature
    T[4] = np.nan
    r = verify_chain(t, d, x, T, u)
    np.testing.assert_array_equal(r["valid"], [True, False, False, False, False, True])
    assert np.all(r["accept_len"][1:5] == -1)
    assert np.all(r["out_tokens"][1:5] == -1)
    assert r["accept_len"][0] >= 0 and r["accept_len"][5] >= 0


def test_timeline_figure(golden_dir):
    # K = 4: positions 0 and 1 have p >= q at the drafted token (always kept),
    # position 2 drafts a token the target gives zero probability (always
    # rejected), so position 3 is discarded and 3 tokens come out.
    g = json.load(open(os.path.join(golden_dir, "timeline_k4.json")))
    K = g["K"]
    V = 6
    rng = _rng(12)
    t = rng.normal(0, 1, (1, K + 1, V))
    d = t[:, :K].copy()
    x = np.array([[1, 2, 3, 4]])
    t[0, 0, 1] = d[0, 0, 1] + 1.0   # p(x) > q(x)
    t[0, 1, 2] = d[0, 1, 2] + 2.0
    t[0, 2, 3] = -5000.0            # p(x) = 0 -> alpha = 0
    for u0 in (0.0, 0.3, 0.9999999):
        r = verify_chain(t, d, x, np.ones(1), np.full((1, K + 1), u0))
        decisions = ["accept" if k < r["accept_len"][0] else ("reject" if k == r["accept_len"][0] else "discard")
                     for k in range(K)]
        assert decisions == g["decisions"]
        assert r["accept_len"][0] == g["replacement_position"]
        assert int((r["out_tokens"][0] >= 0).sum()) == g["net_yield_tokens"]
        assert r["out_tokens"][0, 2] != 3  # the replacement is never the rejected token here
