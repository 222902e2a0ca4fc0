"""Statistical pins for the chain oracle (Monte Carlo, 10^6 seeded trials each).

* Accept-length law: with the same (p, q) at every position and x ~ q, the
  number of accepted drafts is capped-geometric with rate sum_x min(p, q), and
  the mean tokens per iteration equals (1 - alpha^(K+1)) / (1 - alpha); the
  page's worked example prints 2.8 and 4.1 for alpha = 0.7 / 0.9 at K = 4.
* Losslessness: the token emitted at position k (given the run reaches k) is
  distributed as p_k, checked with a chi-square test; two planted mistakes in
  the oracle (resampling from p instead of the residual; accepting when
  u < p(x)) must fail the same test.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.specverify_oracle as ov
from oracle import temperature_softmax, verify_chain
from workloads import MC_CONFIG, mc_chain_inputs

TRIALS = 1_000_000
CHUNK = 200_000


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


def _run_chunks(target_row, draft_row, tokens, T, u):
    n = tokens.shape[0]
    K1, V = target_row.shape
    out_j = np.empty(n, np.int64)
    out_t = np.empty((n, K1), np.int64)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        m = e - s
        r = verify_chain(np.broadcast_to(target_row, (m, K1, V)), np.broadcast_to(draft_row, (m, K1 - 1, V)),
                         tokens[s:e], T[s:e], u[s:e])
        out_j[s:e] = r["accept_len"]
        out_t[s:e] = r["out_tokens"]
    return out_j, out_t


def _chi2_pvalue(counts, probs):
    """Pearson chi-square p-value, merging bins with expected count < 5."""
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    obs_m, exp_m = [], []
    acc_o = acc_e = 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= 5:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        if exp_m:
            obs_m[-1] += acc_o
            exp_m[-1] += acc_e
        else:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
    obs_m = np.array(obs_m)
    exp_m = np.array(exp_m)
    if len(obs_m) < 2:
        return 1.0
    return float(stats.chisquare(obs_m, exp_m * obs_m.sum() / exp_m.sum()).pvalue)


def _two_token_pair(alpha):
    # p = (alpha - 0.1, 1.1 - alpha), q = (0.9, 0.1): sum min(p, q) = alpha.
    p = np.array([alpha - 0.1, 1.1 - alpha])
    q = np.array([0.9, 0.1])
    return np.log(p), np.log(q), p, q


@pytest.mark.slow
@pytest.mark.parametrize("case", [0, 1])
def test_accept_length_law_and_expected_tokens(case, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "expected_tokens_per_iteration.json")))
    c = g["cases"][case]
    alpha, K = c["alpha"], c["gamma"]
    lp, lq, p, q = _two_token_pair(alpha)
    assert np.minimum(p, q).sum() == pytest.approx(alpha, abs=1e-15)
    rng = _rng(100 + case)
    target_row = np.tile(lp, (K + 1, 1))
    draft_row = np.tile(lq, (K, 1))
    tokens = (rng.random((TRIALS, K)) >= q[0]).astype(np.int64)  # x ~ q at every position
    u = rng.random((TRIALS, K + 1))
    T = np.ones(TRIALS)
    j, _ = _run_chunks(target_row, draft_row, tokens, T, u)
    # capped geometric law of the accepted-prefix length
    law = np.array([alpha ** n * (1 - alpha) for n in range(K)] + [alpha ** K])
    counts = np.bincount(j, minlength=K + 1)
    assert _chi2_pvalue(counts, law) > 0.01
    # mean tokens per iteration vs the closed form, and the closed form vs the page
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    tokens_per_iter = j + 1
    se = tokens_per_iter.std() / np.sqrt(TRIALS)
    assert abs(tokens_per_iter.mean() - closed) < 4 * se
    assert round(closed, g["printed_decimals"]) == c["printed"]


def _mc_inputs():
    x = mc_chain_inputs(MC_CONFIG, TRIALS)
    tr = x["target_row"].double().numpy()
    dr = x["draft_row"].double().numpy()
    return tr, dr, x["draft_tokens"].numpy().astype(np.int64), x["temperature"].double().numpy(), \
        x["uniforms"].double().numpy()


def _lossless_pvalues(tr, dr, tokens, T, u):
    j, out = _run_chunks(tr, dr, tokens, T, u)
    K1, V = tr.shape
    p = temperature_softmax(tr, np.full(K1, T[0]))
    pvals = []
    for k in range(K1):
        sel = j >= k
        counts = np.bincount(out[sel, k], minlength=V)
        pvals.append(_chi2_pvalue(counts, p[k]))
    return pvals, j


@pytest.fixture(scope="module")
def mc_inputs():
    return _mc_inputs()


@pytest.mark.slow
def test_emitted_tokens_follow_target_distribution(mc_inputs):
    tr, dr, tokens, T, u = mc_inputs
    # the draft really is x ~ q (the generator side of the experiment)
    q = temperature_softmax(dr, np.full(dr.shape[0], T[0]))
    for k in range(dr.shape[0]):
        assert _chi2_pvalue(np.bincount(tokens[:, k], minlength=dr.shape[1]), q[k]) > 1e-4
    pvals, j = _lossless_pvalues(tr, dr, tokens, T, u)
    assert min(pvals) > 0.01, pvals
    # the draft differs enough from the target for rejections to matter
    assert 0.05 < (j < dr.shape[0]).mean() < 0.95


@pytest.mark.slow
def test_negative_control_resample_from_p_fails(mc_inputs, monkeypatch):
    monkeypatch.setattr(ov, "residual_weights", lambda p, q: np.asarray(p, np.float64).copy())
    pvals, _ = _lossless_pvalues(*mc_inputs)
    assert min(pvals) < 1e-6, pvals


@pytest.mark.slow
def test_negative_control_accept_if_u_below_p_fails(mc_inputs, monkeypatch):
    monkeypatch.setattr(ov, "acceptance_probability", lambda p_x, q_x: np.asarray(p_x, np.float64))
    pvals, _ = _lossless_pvalues(*mc_inputs)
    assert min(pvals) < 1e-6, pvals


@pytest.mark.slow
def test_negative_control_reused_uniform_fails(mc_inputs):
    # Drawing the replacement with the uniform that just failed its accept test
    # (instead of the separate last column) biases the residual draw.
    tr, dr, tokens, T, u = mc_inputs
    K = dr.shape[0]
    j_first, _ = _run_chunks(tr, dr, tokens, T, u)
    u2 = u.copy()
    rows = np.flatnonzero(j_first < K)
    u2[rows, K] = u[rows, j_first[rows]]
    pvals, _ = _lossless_pvalues(tr, dr, tokens, T, u2)
    assert min(pvals) < 1e-6, pvals


def test_oracle_module_exports():
    assert oracle.FLAG_WINDOW == 1e-6


def test_flag_rate_predicts_the_flagged_count():
    """The oracle's flag_rate diagnostic (the chance that fresh uniforms land
    within the 1e-6 window of a decision threshold) predicts how many rows
    are flagged: over 2 x 10^6 seeded trials of the V = 16, K = 3 workload
    (fresh uniforms for each million) the flagged count is a Poisson count
    with mean sum(flag_rate). With V = 16 about 3e-5 of the rows flag, so the
    count is large enough to test; a rate off by a factor of two (one side
    of each window only, say) fails by more than 5 sigma."""
    from workloads.synth import seed_stream

    x = mc_chain_inputs(MC_CONFIG, TRIALS)
    tr = x["target_row"].double().numpy()
    dr = x["draft_row"].double().numpy()
    tokens = x["draft_tokens"].numpy().astype(np.int64)
    T = x["temperature"].double().numpy()
    K1, V = tr.shape
    flagged = rate = 0.0
    for it in (1, 2):
        u = seed_stream(MC_CONFIG.config_id, MC_CONFIG.variant, 3, 100 + it).random((TRIALS, K1), dtype=np.float32)
        u = u.astype(np.float64)
        for s in range(0, TRIALS, CHUNK):
            e = min(TRIALS, s + CHUNK)
            m = e - s
            r = verify_chain(np.broadcast_to(tr, (m, K1, V)), np.broadcast_to(dr, (m, K1 - 1, V)), tokens[s:e],
                             T[s:e], u[s:e])
            flagged += float(r["flagged"].sum())
            rate += float(r["flag_rate"].sum())
    assert rate > 40, rate
    z = (flagged - rate) / np.sqrt(rate)
    print("flagged", flagged, "expected", rate, "z", z)
    assert abs(z) < 5, (flagged, rate)
