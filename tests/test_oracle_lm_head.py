"""Pins of the oracle's LM-head step: logits = hidden x weight^T in float64,
stored as bfloat16, then chain verification on them.

* bfloat16 rounding against PyTorch's float32 -> bfloat16 conversion (round
  to nearest, ties to even) on float32 values, ties placed on purpose;
* the float64 matmul against math.fsum of the exact products on sampled
  elements (products of bfloat16 values are exact in float64, so fsum gives
  the correctly rounded sum), with planted mistakes (a transposed weight, a
  dropped last column) that the same check catches;
* an integer case where every sum is an exact integer;
* the composition: verify_chain_lm_head equals verify_chain on the rounded
  logits.
"""
import math

import numpy as np
import torch

import oracle


def _rng(seed):
    return np.random.Generator(np.random.Philox(seed))


def _bf16_grid(rng, shape, scale):
    """Values that bfloat16 holds exactly (random normals rounded by torch)."""
    return torch.from_numpy(rng.normal(0.0, scale, shape).astype(np.float32)).to(torch.bfloat16).double().numpy()


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = _rng(1)
    x = (rng.normal(0, 1, 200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)), ref)


def test_round_to_bf16_ties_go_to_even():
    # m in [1, 2) with 7 fraction bits kept; a value exactly halfway between
    # two neighbours (the eighth fraction bit set, nothing below) goes to the
    # one whose last kept bit is 0
    base = np.arange(128, 256, dtype=np.float64) / 128.0  # every bfloat16 mantissa in [1, 2)
    halfway = base + 2.0 ** -8
    got = oracle.round_to_bf16(np.concatenate([halfway, -halfway, halfway * 2.0 ** 40]))
    k = np.arange(128, 256)
    up = (k % 2 == 1)  # an odd last bit rounds up to the even neighbour
    want = np.where(up, base + 2.0 ** -7, base)
    np.testing.assert_array_equal(got, np.concatenate([want, -want, want * 2.0 ** 40]))
    ref = torch.from_numpy(halfway.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got[:128], ref)


def test_round_to_bf16_keeps_representable_values_and_zero():
    rng = _rng(2)
    v = _bf16_grid(rng, 5000, 3.0)
    np.testing.assert_array_equal(oracle.round_to_bf16(v), v)
    assert oracle.round_to_bf16(0.0) == 0.0
    np.testing.assert_array_equal(oracle.round_to_bf16([-np.inf, np.inf]), [-np.inf, np.inf])


def _fsum_logit(hidden, weight, m, v):
    return math.fsum(float(a) * float(b) for a, b in zip(hidden[m], weight[v]))


def test_lm_head_logits_against_exact_sums():
    rng = _rng(3)
    M, H, V = 24, 1024, 3000
    hidden = _bf16_grid(rng, (M, H), 1.0)
    weight = _bf16_grid(rng, (V, H), 2.5 / math.sqrt(H))
    got = oracle.lm_head_logits(hidden, weight)
    assert got.shape == (M, V)
    mi = rng.integers(0, M, 300)
    vi = rng.integers(0, V, 300)
    exact = np.array([_fsum_logit(hidden, weight, m, v) for m, v in zip(mi, vi)])
    scale = np.array([np.sum(np.abs(hidden[m] * weight[v])) for m, v in zip(mi, vi)])
    # float64 summation of H exact products: error below H * 2^-53 * sum |products|
    assert np.all(np.abs(got[mi, vi] - exact) <= H * 2.0 ** -53 * scale)
    # planted mistakes the same check sees: the weight used transposed in its
    # square block, and the last hidden column dropped
    wrong = oracle.lm_head_logits(hidden[:, :H], weight[:, ::-1])
    assert np.any(np.abs(wrong[mi, vi] - exact) > 1e-6)
    dropped = oracle.lm_head_logits(hidden[:, :-1], weight[:, :-1])
    assert np.any(np.abs(dropped[mi, vi] - exact) > 1e-9)


def test_lm_head_logits_integer_case_is_exact():
    rng = _rng(4)
    M, H, V = 12, 8192, 500
    hidden = rng.integers(-3, 4, (M, H)).astype(np.float64)
    weight = rng.integers(-3, 4, (V, H)).astype(np.float64)
    got = oracle.lm_head_logits(hidden, weight)
    want = (hidden.astype(np.int64) @ weight.astype(np.int64).T).astype(np.float64)
    np.testing.assert_array_equal(got, want)
    # and below 2^24 in magnitude, so a float32 accumulation is exact too
    assert np.abs(want).max() < 2 ** 24


def test_verify_chain_lm_head_is_verify_chain_on_the_stored_logits():
    rng = _rng(5)
    B, K, H, V = 6, 3, 256, 700
    hidden = _bf16_grid(rng, (B, K + 1, H), 1.0)
    weight = _bf16_grid(rng, (V, H), 3.0 / math.sqrt(H))
    t64 = oracle.round_to_bf16(oracle.lm_head_logits(hidden, weight))
    draft = _bf16_grid(rng, (B, K, V), 1.0) + t64[:, :K]
    tokens = rng.integers(0, V, (B, K))
    T = rng.uniform(0.5, 1.5, B)
    u = rng.random((B, K + 1))
    got = oracle.verify_chain_lm_head(hidden, weight, draft, tokens, T, u)
    want = oracle.verify_chain(t64, draft, tokens, T, u)
    np.testing.assert_array_equal(got["target_logits"], t64)
    for k in ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass"):
        np.testing.assert_array_equal(got[k], want[k])
    # the stored logits are bfloat16 values
    np.testing.assert_array_equal(oracle.round_to_bf16(got["target_logits"]), got["target_logits"])
