"""GPU parity of the LM-head calls: sv_lm_head_logits and sv_verify_chain_lm_head.

* Integer hidden states and weights in [-3, 3]: every sum is an integer below
  2^24, so the kernel's fp32 accumulation is exact in any order; the stored
  bf16 logits must equal the oracle's (fp64 matmul, then round to nearest
  even) bit for bit, and the verification outputs must match the oracle's
  verification on those logits as in every chain parity test (tokens exact
  outside the flag window, probabilities to 1e-5). This covers the
  epilogue's statistics, the combine of the pieces, the draft-row stream and
  the draw, at ragged small shapes and at the full B=64 K=5 V=128256 H=8192.
* Real-valued weights: the logits must lie within the fp32 accumulation
  bound of the oracle's fp64 logits (plus half a bf16 ulp); and the call
  must agree with sv_verify_chain run on the logits it returned (the same
  verification from the stored logits, statistics from the stream instead
  of the epilogue).
Every case prints its name and shape before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (REL_TOL, ChainReport, assert_chain_parity, check_chain_structure, compare_chain,
                    oracle_chain_chunked, record_parity, to_np64, to_np_i)
from workloads import LM_HEAD_CONFIGS, lm_head_chain_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _int_operands(seed, M, H, V):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hidden = torch.randint(-3, 4, (M, H), generator=g, device="cuda").to(torch.bfloat16)
    weight = torch.randint(-3, 4, (V, H), generator=g, device="cuda").to(torch.bfloat16)
    return hidden, weight


def _oracle_logits(hidden, weight, v_chunk=8192):
    """The oracle's logits, a chunk of vocabulary rows at a time (fp64)."""
    h = to_np64(hidden.reshape(-1, hidden.shape[-1]))
    parts = [oracle.lm_head_logits(h, to_np64(weight[v0:v0 + v_chunk])) for v0 in range(0, weight.shape[0], v_chunk)]
    return np.concatenate(parts, axis=1)


@pytest.mark.parametrize("M,H,V", [(37, 64, 1000), (128, 256, 1024), (200, 512, 4104), (384, 8192, 2048)])
def test_lm_head_logits_integer_exact(sv, M, H, V):
    _say("lm head logits, integer operands", (M, H, V))
    hidden, weight = _int_operands(100 + M + V, M, H, V)
    got = sv.sv_lm_head_logits(hidden, weight)
    torch.cuda.synchronize()
    want = oracle.round_to_bf16(_oracle_logits(hidden, weight))
    np.testing.assert_array_equal(to_np64(got), want)


def _ulp_bf16(x):
    x = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(x)).astype(np.int64) - 7)


def _logits_within_bound(got, hidden, weight, rows):
    """|stored - fp64| <= half a bf16 ulp + H 2^-24 sum_h |hidden weight| on `rows`."""
    h = to_np64(hidden.reshape(-1, hidden.shape[-1]))[rows]
    g_all = got.reshape(-1, weight.shape[0])[torch.from_numpy(rows).to(got.device)]
    worst, nflip, n = 0.0, 0, 0
    for v0 in range(0, weight.shape[0], 16384):  # a chunk of vocabulary rows at a time
        w = to_np64(weight[v0:v0 + 16384])
        ref = oracle.lm_head_logits(h, w)
        acc = weight.shape[1] * 2.0 ** -24 * (np.abs(h) @ np.abs(w).T)
        g = to_np64(g_all[:, v0:v0 + 16384])
        bound = 0.5 * _ulp_bf16(np.abs(ref) + acc) + acc
        err = np.abs(g - ref)
        assert np.all(err <= bound), f"worst excess {np.max(err - bound)}"
        worst = max(worst, float(err.max()))
        nflip += int(np.sum(g != oracle.round_to_bf16(ref)))
        n += g.size
    return worst, nflip / n


def test_lm_head_logits_real_within_the_accumulation_bound(sv):
    M, H, V = 96, 1024, 3000
    _say("lm head logits, real operands", (M, H, V))
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    hidden = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
    weight = (torch.randn((V, H), generator=g, device="cuda") * (2.5 / math.sqrt(H))).to(torch.bfloat16)
    got = sv.sv_lm_head_logits(hidden, weight)
    torch.cuda.synchronize()
    err, flips = _logits_within_bound(got, hidden, weight, np.arange(M))
    print("max |err|", err, "bf16 values that differ from rounding the fp64 logit:", flips, flush=True)
    assert flips < 0.01


def _fused(sv, x, **kw):
    out = sv.sv_verify_chain_lm_head(x["hidden"], x["weight"], x["draft"], x["draft_tokens"], x["temperature"],
                                     x["uniforms"], **kw)
    torch.cuda.synchronize()
    return out


def _parity_integer(sv, cfg, record=None):
    x = lm_head_chain_inputs(cfg, device="cuda")
    out = _fused(sv, x)
    assert int(out["err_flags"].item()) == 0
    check_chain_structure(out, cfg.K, cfg.V)
    t = oracle.round_to_bf16(_oracle_logits(x["hidden"], x["weight"])).reshape(cfg.B, cfg.K + 1, cfg.V)
    np.testing.assert_array_equal(to_np64(out["target_logits"]), t)
    inp = {"target": torch.from_numpy(t).to(torch.bfloat16), "draft": x["draft"].cpu(),
           "draft_tokens": x["draft_tokens"].cpu(), "temperature": x["temperature"].cpu(),
           "uniforms": x["uniforms"].cpu()}
    (ref,) = oracle_chain_chunked(inp, [inp["uniforms"]])
    rep = compare_chain(out, ref)
    print(cfg.name, rep, flush=True)
    if record:
        record_parity(record, call="sv_verify_chain_lm_head", logits_bit_exact=True, **rep.record())
    assert_chain_parity(rep)
    return out, rep


@pytest.mark.parametrize("B,K,V,H", [(6, 3, 2048, 256), (5, 4, 1000, 64), (3, 0, 4104, 128), (40, 2, 10000, 512)])
def test_fused_chain_integer_small(sv, B, K, V, H):
    cfg = LM_HEAD_CONFIGS["c2h_int"].with_(B=B, K=K, V=V, H=H, variant=B + K)
    _say("fused lm head chain, integer", cfg.name, (B, K, V, H))
    _parity_integer(sv, cfg)


def test_fused_chain_integer_full_shape(sv):
    cfg = LM_HEAD_CONFIGS["c2h_int"]
    _say("fused lm head chain, integer, full shape", cfg.name, (cfg.B, cfg.K, cfg.V, cfg.H))
    _, rep = _parity_integer(sv, cfg, record=cfg.name)
    assert rep.rows == cfg.B and 0.2 < rep.mean_alpha < 0.98


def test_fused_chain_real_weights(sv):
    cfg = LM_HEAD_CONFIGS["c2h"]
    _say("fused lm head chain, real weights", cfg.name, (cfg.B, cfg.K, cfg.V, cfg.H))
    x = lm_head_chain_inputs(cfg, device="cuda")
    out = _fused(sv, x)
    assert int(out["err_flags"].item()) == 0
    check_chain_structure(out, cfg.K, cfg.V)
    # the stored logits: within the accumulation bound of the fp64 logits (sampled rows)
    rows = np.arange(0, cfg.B * (cfg.K + 1), 24)
    err, flips = _logits_within_bound(out["target_logits"], x["hidden"], x["weight"], rows)
    print("stored logits: max |err|", err, "rounding flips", flips, flush=True)
    # the same verification from the stored logits through the stream path
    plain = sv.sv_verify_chain(out["target_logits"], x["draft"], x["draft_tokens"], x["temperature"], x["uniforms"])
    torch.cuda.synchronize()
    for k in ("p_draft", "q_draft"):
        a, b = to_np64(out[k]), to_np64(plain[k])
        assert np.all(np.abs(a - b) <= REL_TOL * np.abs(b) + 1e-30), k
    same = (to_np_i(out["accept_len"]) == to_np_i(plain["accept_len"])) & np.all(
        to_np_i(out["out_tokens"]) == to_np_i(plain["out_tokens"]), axis=1)
    alpha = np.minimum(1.0, to_np64(out["p_draft"]) / np.maximum(to_np64(out["q_draft"]), 1e-300))
    near = np.any(np.abs(to_np64(x["uniforms"])[:, :cfg.K] - alpha) < 1e-6, axis=1)
    print("rows", cfg.B, "identical", int(same.sum()), "near an accept threshold", int(near.sum()), flush=True)
    # the draw's boundaries are not known without the oracle: allow a few near-boundary draws
    assert int((~same & ~near).sum()) <= 2
    record_parity(cfg.name, call="sv_verify_chain_lm_head (real weights)", rows=cfg.B,
                  stored_logits_max_abs_err=err, rounding_flips=flips,
                  rows_identical_to_sv_verify_chain_on_the_stored_logits=int(same.sum()))


def test_fused_workspace_returns_to_zero_and_errors(sv):
    cfg = LM_HEAD_CONFIGS["c2h_int"].with_(B=8, K=3, V=4096, H=128, variant=71)
    _say("fused lm head chain: workspace and data errors", (cfg.B, cfg.K, cfg.V, cfg.H))
    x = lm_head_chain_inputs(cfg, device="cuda")
    ws = torch.zeros(sv.sv_lm_head_chain_workspace_bytes(cfg.B, cfg.K, cfg.V, cfg.H), dtype=torch.uint8,
                     device="cuda")
    _fused(sv, x, workspace_tensor=ws)
    assert int(ws.count_nonzero().item()) == 0
    x["draft_tokens"][1, 0] = cfg.V
    x["temperature"][2] = 0.0
    out = _fused(sv, x, workspace_tensor=ws)
    flags = int(out["err_flags"].item())
    assert flags & sv.SV_ERRF_TOKEN and flags & sv.SV_ERRF_TEMPERATURE
    acc = to_np_i(out["accept_len"])
    assert acc[1] == -1 and acc[2] == -1 and np.all(np.delete(acc, [1, 2]) >= 0)
    assert int(ws.count_nonzero().item()) == 0
