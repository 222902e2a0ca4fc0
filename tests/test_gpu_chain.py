"""GPU parity of sv_verify_chain against the CPU oracle (run on an MI355X).

Every case prints its name, shape and seed before touching the GPU.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from parity import (
    ChainReport,
    assert_chain_parity,
    check_chain_structure,
    compare_chain,
    oracle_chain,
    oracle_chain_chunked,
    record_parity,
    to_np_i,
)
from workloads import CHAIN_CONFIGS, MC_CONFIG, chain_inputs, mc_chain_inputs
from workloads.synth import chain_uniforms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _to(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _run(sv, inp, **kw):
    out = sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                             inp["uniforms"], **kw)
    torch.cuda.synchronize()
    return out


def _parity_full(sv, inp_dev, label):
    _say(label, tuple(inp_dev["target"].shape), inp_dev["target"].dtype)
    out = _run(sv, inp_dev)
    K, V = inp_dev["target"].shape[1] - 1, inp_dev["target"].shape[2]
    check_chain_structure(out, K, V)
    ref = oracle_chain(inp_dev)
    rep = compare_chain(out, ref)
    print(label, rep, flush=True)
    assert int(out["err_flags"].item()) == 0
    assert_chain_parity(rep)
    return out, ref, rep


# ----------------------------------------------------------------------------- the workloads

def test_c1_full(sv):
    cfg = CHAIN_CONFIGS["c1"]
    _, _, rep = _parity_full(sv, _to(chain_inputs(cfg), "cuda"), cfg.name)
    record_parity(cfg.name, call="sv_verify_chain", **rep.record())


def test_c1_recipe_more_sequences(sv):
    cfg = CHAIN_CONFIGS["c1"].with_(B=128, variant=7)
    _parity_full(sv, _to(chain_inputs(cfg), "cuda"), cfg.name + "_b128")


@pytest.mark.parametrize("B,K", [(1, 5), (4, 5), (16, 5), (2, 8), (23, 5)])
def test_small_calls_at_the_c2_row_shape(sv, B, K):
    # the pages' batch sizes (1 to 16 sequences) at V = 128256 bf16: calls of
    # at most 256 rows in all take the small form (one launch whose
    # statistics workgroups decide and draw), compared in full
    cfg = CHAIN_CONFIGS["c2"].with_(B=B, K=K, variant=40 + B + K)
    assert sv.sv_chain_form(B, K, cfg.V, torch.bfloat16) == 1
    inp = chain_inputs(cfg, device="cuda")
    _, _, rep = _parity_full(sv, inp, f"{cfg.name} small call B={B} K={K}")
    record_parity(f"{cfg.name}_small_b{B}_k{K}", call="sv_verify_chain (small form)", **rep.record())


def test_c2_full(sv):
    cfg = CHAIN_CONFIGS["c2"]
    inp = chain_inputs(cfg, device="cuda")
    _, ref, rep = _parity_full(sv, inp, cfg.name)
    record_parity(cfg.name, call="sv_verify_chain", **rep.record())
    assert 0.3 < rep.mean_alpha < 0.95


@pytest.mark.parametrize("key", ["c3_s0.3", "c3_s1.0", "c3_s3.0"])
def test_c3_full(sv, key):
    """Every one of the 256 sequences of each divergence, against the oracle."""
    cfg = CHAIN_CONFIGS[key]
    _say(cfg.name, (cfg.B, cfg.K + 1, cfg.V))
    inp = chain_inputs(cfg, device="cuda")
    out = _run(sv, inp)
    check_chain_structure(out, cfg.K, cfg.V)
    assert int(out["err_flags"].item()) == 0
    (ref,) = oracle_chain_chunked(inp, [inp["uniforms"]])
    rep = compare_chain(out, ref)
    print(cfg.name, rep, flush=True)
    assert rep.rows == cfg.B
    record_parity(cfg.name, call="sv_verify_chain", **rep.record())
    assert_chain_parity(rep)
    # acceptance falls as the draft drifts from the target
    j = to_np_i(out["accept_len"])
    print(cfg.name, "mean accept_len", j.mean(), flush=True)


def test_c5_ten_iterations_full(sv):
    """All 1024 sequences of all ten back-to-back iterations against the
    oracle; the oracle forms each sequence's distributions once and verifies
    them with the ten sets of uniforms (every decision and draw is its own)."""
    cfg = CHAIN_CONFIGS["c5"]
    _say(cfg.name, (cfg.B, cfg.K + 1, cfg.V), "iterations", cfg.iterations)
    inp = chain_inputs(cfg, device="cuda")
    uni = [chain_uniforms(cfg, it, "cuda") for it in range(cfg.iterations)]
    outs = []
    for it in range(cfg.iterations):  # back to back on one stream
        outs.append(sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"], uni[it]))
    torch.cuda.synchronize()
    for it in range(cfg.iterations):
        check_chain_structure(outs[it], cfg.K, cfg.V)
        assert int(outs[it]["err_flags"].item()) == 0
    _say(cfg.name, "oracle over every sequence of the ten iterations")
    refs = oracle_chain_chunked(inp, uni)
    total = ChainReport()
    for it in range(cfg.iterations):
        total = total.merge(compare_chain(outs[it], refs[it]))
    print(cfg.name, total, flush=True)
    assert total.rows == cfg.B * cfg.iterations
    record_parity(cfg.name, call="sv_verify_chain", iterations=cfg.iterations, **total.record())
    assert_chain_parity(total)


def test_mc_losslessness_on_gpu(sv):
    n = MC_CONFIG.B
    _say(MC_CONFIG.name, "trials", n)
    x = mc_chain_inputs(MC_CONFIG, n)
    K, V = MC_CONFIG.K, MC_CONFIG.V
    inp = {
        "target": x["target_row"].expand(n, K + 1, V).contiguous().cuda(),
        "draft": x["draft_row"].expand(n, K, V).contiguous().cuda(),
        "draft_tokens": x["draft_tokens"].cuda(),
        "temperature": x["temperature"].cuda(),
        "uniforms": x["uniforms"].cuda(),
    }
    out = _run(sv, inp)
    check_chain_structure(out, K, V)
    j = to_np_i(out["accept_len"])
    toks = to_np_i(out["out_tokens"])
    # element-wise parity with the oracle, in chunks
    total = ChainReport()
    for s in range(0, n, 200_000):
        rows = np.arange(s, min(n, s + 200_000))
        ref = oracle_chain(inp, torch.from_numpy(rows))
        total = total.merge(compare_chain(out, ref, rows))
    print(MC_CONFIG.name, total, flush=True)
    assert_chain_parity(total)
    # the GPU's emitted tokens follow p at every position
    tr = x["target_row"].double().numpy()
    p = oracle.temperature_softmax(tr, np.ones(K + 1))
    pvalues = []
    for k in range(K + 1):
        sel = j >= k
        counts = np.bincount(toks[sel, k], minlength=V)
        exp = p[k] * sel.sum()
        keep = exp >= 5
        obs = np.append(counts[keep], counts[~keep].sum())
        ex = np.append(exp[keep], exp[~keep].sum())
        if ex[-1] == 0:
            obs, ex = obs[:-1], ex[:-1]
        pv = stats.chisquare(obs, ex * obs.sum() / ex.sum()).pvalue
        print("position", k, "chi2 p", pv, flush=True)
        pvalues.append(pv)
    record_parity(MC_CONFIG.name, call="sv_verify_chain", chi2_pvalues_per_position=pvalues, **total.record())
    assert min(pvalues) > 0.01


# ----------------------------------------------------------------------------- edge cases

def _rand_case(B, K, V, dtype, seed, sigma_t=3.0, sigma_d=1.0, T=None, tokens_from_q=True):
    g = np.random.Generator(np.random.Philox(seed))
    t64 = g.standard_normal((B, K + 1, V)) * sigma_t
    d64 = t64[:, :K] + g.standard_normal((B, K, V)) * sigma_d
    Tm = np.full(B, 1.0, np.float32) if T is None else np.asarray(T, np.float32)
    target = torch.from_numpy(t64).to(dtype)
    draft = torch.from_numpy(d64).to(dtype)
    if tokens_from_q and K > 0:
        d = draft.double().numpy() / Tm.astype(np.float64)[:, None, None]
        x = np.argmax(d + g.gumbel(size=d.shape), axis=-1)
    else:
        x = g.integers(0, V, (B, K))
    return {
        "target": target,
        "draft": draft,
        "draft_tokens": torch.from_numpy(x.astype(np.int32)),
        "temperature": torch.from_numpy(Tm),
        "uniforms": torch.from_numpy(g.random((B, K + 1), dtype=np.float32)),
    }


EDGE = [
    # B, K, V, dtype
    (64, 3, 1, torch.float32),
    (64, 3, 2, torch.bfloat16),
    (64, 3, 5, torch.bfloat16),
    (64, 2, 8, torch.float32),
    (64, 4, 16, torch.bfloat16),
    (32, 4, 33, torch.float32),
    (32, 4, 2047, torch.bfloat16),
    (32, 4, 2048, torch.bfloat16),
    (32, 4, 2049, torch.float32),
    (16, 5, 32003, torch.bfloat16),
    (16, 5, 32003, torch.float32),
    (8, 1, 50000, torch.bfloat16),
    (4, 63, 1000, torch.bfloat16),
    (16, 0, 5000, torch.bfloat16),
    (3, 2, 300001, torch.bfloat16),
]


@pytest.mark.parametrize("B,K,V,dtype", EDGE, ids=[f"B{b}_K{k}_V{v}_{str(d)[6:]}" for b, k, v, d in EDGE])
def test_edge_shapes(sv, B, K, V, dtype):
    inp = _rand_case(B, K, V, dtype, seed=1000 + V + K)
    if K == 0:
        inp["draft"] = None
        inp["draft_tokens"] = None
    _parity_full(sv, _to(inp, "cuda"), f"edge B{B} K{K} V{V} {dtype}")


@pytest.mark.parametrize("T", [0.05, 0.3, 5.0])
def test_temperature_extremes(sv, T):
    inp = _rand_case(64, 4, 4096, torch.bfloat16, seed=77, T=np.full(64, T))
    _parity_full(sv, _to(inp, "cuda"), f"temperature {T}")


def test_per_row_temperatures(sv):
    g = np.random.Generator(np.random.Philox(5))
    inp = _rand_case(128, 6, 10000, torch.bfloat16, seed=78, T=g.uniform(0.3, 1.3, 128))
    _parity_full(sv, _to(inp, "cuda"), "per-row temperature")


def test_draft_equals_target_accepts_all(sv):
    inp = _rand_case(64, 5, 20000, torch.bfloat16, seed=79)
    inp["draft"] = inp["target"][:, :5].contiguous()
    out, ref, _ = _parity_full(sv, _to(inp, "cuda"), "draft == target")
    assert np.all(to_np_i(out["accept_len"]) == 5)
    assert np.all(out["residual_mass"].cpu().numpy() == -1.0)


def test_disjoint_supports_reject_first(sv):
    B, K, V = 32, 3, 4096
    g = np.random.Generator(np.random.Philox(80))
    t = np.full((B, K + 1, V), -1000.0)
    d = np.full((B, K, V), -1000.0)
    t[:, :, 0::2] = g.standard_normal((B, K + 1, V // 2))
    d[:, :, 1::2] = g.standard_normal((B, K, V // 2))
    x = 2 * g.integers(0, V // 2, (B, K)) + 1
    inp = {
        "target": torch.from_numpy(t).float(),
        "draft": torch.from_numpy(d).float(),
        "draft_tokens": torch.from_numpy(x.astype(np.int32)),
        "temperature": torch.ones(B),
        "uniforms": torch.from_numpy(g.random((B, K + 1), dtype=np.float32)),
    }
    out, _, _ = _parity_full(sv, _to(inp, "cuda"), "disjoint supports")
    assert np.all(to_np_i(out["accept_len"]) == 0)
    assert np.all(to_np_i(out["out_tokens"])[:, 0] % 2 == 0)
    np.testing.assert_allclose(out["residual_mass"].cpu().numpy(), 1.0, rtol=1e-5)


def test_empty_batch(sv):
    inp = _rand_case(0, 3, 100, torch.bfloat16, seed=81)
    out = _run(sv, _to(inp, "cuda"))
    assert out["accept_len"].numel() == 0


def test_without_optional_outputs(sv):
    inp = _to(_rand_case(16, 4, 3000, torch.bfloat16, seed=82), "cuda")
    _say("no optional outputs")
    a = _run(sv, inp, want_probs=False)
    b = _run(sv, inp)
    assert torch.equal(a["accept_len"], b["accept_len"]) and torch.equal(a["out_tokens"], b["out_tokens"])


def test_default_temperature_is_one(sv):
    inp = _to(_rand_case(16, 4, 3000, torch.bfloat16, seed=83), "cuda")
    _say("temperature NULL")
    a = _run(sv, {**inp, "temperature": None})
    b = _run(sv, inp)
    assert torch.equal(a["out_tokens"], b["out_tokens"])


def test_data_errors_are_flagged_per_row(sv):
    inp = _rand_case(8, 3, 1000, torch.bfloat16, seed=84)
    inp["draft_tokens"][1, 2] = 1000
    inp["draft_tokens"][2, 0] = -5
    inp["temperature"][3] = 0.0
    inp["temperature"][4] = float("nan")
    inp["temperature"][5] = -1.0
    _say("data errors")
    out = _run(sv, _to(inp, "cuda"))
    flags = int(out["err_flags"].item())
    assert flags & sv.SV_ERRF_TOKEN and flags & sv.SV_ERRF_TEMPERATURE
    j = to_np_i(out["accept_len"])
    assert np.all(j[1:6] == -1) and np.all(to_np_i(out["out_tokens"])[1:6] == -1)
    good = [0, 6, 7]
    ref = oracle_chain(inp, good)
    rep = compare_chain(out, ref, good)
    assert rep.mismatched_unflagged == 0


def test_repeat_is_bit_identical(sv):
    cfg = CHAIN_CONFIGS["c2"]
    inp = chain_inputs(cfg, device="cuda")
    _say("determinism", cfg.name)
    first = _run(sv, inp)
    for _ in range(10):
        again = _run(sv, inp)
        for k in ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass"):
            assert torch.equal(first[k], again[k]), k


def test_concurrent_one_launch_calls(sv):
    # two calls large enough for the one-launch kernel, on two streams at
    # once (each with its own workspace): together they hold more workgroups
    # than the device, and both must match their single-stream outputs
    cfg = CHAIN_CONFIGS["c2"]
    inp_a = chain_inputs(cfg, device="cuda")
    inp_b = chain_inputs(cfg.with_(variant=cfg.variant + 20, B=96), device="cuda")
    _say("two one-launch calls on two streams", cfg.name, "and B=96 variant", cfg.variant + 20)
    ref_a = _run(sv, inp_a)
    ref_b = _run(sv, inp_b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(5):
        oa = sv.sv_verify_chain(inp_a["target"], inp_a["draft"], inp_a["draft_tokens"], inp_a["temperature"],
                                inp_a["uniforms"], stream=s1)
        ob = sv.sv_verify_chain(inp_b["target"], inp_b["draft"], inp_b["draft_tokens"], inp_b["temperature"],
                                inp_b["uniforms"], stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert int(oa["err_flags"].item()) == 0 and int(ob["err_flags"].item()) == 0
        for k in ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass"):
            assert torch.equal(oa[k], ref_a[k]), k
            assert torch.equal(ob[k], ref_b[k]), k
    assert_chain_parity(compare_chain(ref_b, oracle_chain(inp_b)))


def test_concurrent_streams(sv):
    inp_a = _to(_rand_case(32, 5, 50000, torch.bfloat16, seed=85), "cuda")
    inp_b = _to(_rand_case(48, 4, 30000, torch.float32, seed=86), "cuda")
    _say("two streams")
    ref_a = _run(sv, inp_a)
    ref_b = _run(sv, inp_b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(5):
        with torch.cuda.stream(s1):
            oa = sv.sv_verify_chain(inp_a["target"], inp_a["draft"], inp_a["draft_tokens"], inp_a["temperature"],
                                    inp_a["uniforms"], stream=s1)
        with torch.cuda.stream(s2):
            ob = sv.sv_verify_chain(inp_b["target"], inp_b["draft"], inp_b["draft_tokens"], inp_b["temperature"],
                                    inp_b["uniforms"], stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa["out_tokens"], ref_a["out_tokens"])
        assert torch.equal(ob["out_tokens"], ref_b["out_tokens"])


def test_small_calls_beside_other_launches(sv):
    # Small-form calls (every workgroup of a sequence waits for the sequence's
    # slots) on two streams at once, beside a one-launch call on a third
    # stream that holds more workgroups than the device: every output must
    # equal the same call's on one stream, with no error flag.
    c1 = CHAIN_CONFIGS["c1"]
    inp_a = chain_inputs(c1, device="cuda")
    inp_b = chain_inputs(CHAIN_CONFIGS["c2"].with_(B=16, variant=CHAIN_CONFIGS["c2"].variant + 30), device="cuda")
    inp_c = chain_inputs(CHAIN_CONFIGS["c2"], device="cuda")
    assert sv.sv_chain_form(c1.B, c1.K, c1.V, inp_a["target"].dtype) == 1
    assert sv.sv_chain_form(16, CHAIN_CONFIGS["c2"].K, CHAIN_CONFIGS["c2"].V, torch.bfloat16) == 1
    _say("two small calls and a one-launch call on three streams", c1.name, "B=16 c2 recipe", CHAIN_CONFIGS["c2"].name)
    refs = [_run(sv, inp) for inp in (inp_a, inp_b, inp_c)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = []
    for _ in range(8):
        row = []
        for inp, st in zip((inp_c, inp_a, inp_b), (streams[2], streams[0], streams[1])):
            with torch.cuda.stream(st):
                row.append(sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                                              inp["uniforms"], stream=st))
        outs.append((row[1], row[2], row[0]))
    torch.cuda.synchronize()
    for got in outs:
        for o, ref in zip(got, refs):
            assert int(o["err_flags"].item()) == 0
            for k in ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass"):
                assert torch.equal(o[k], ref[k]), k
    assert_chain_parity(compare_chain(refs[0], oracle_chain(inp_a)))


def test_vanished_residual_draws_from_p(sv):
    """A rejected position whose residual max(0, p - q) sums to zero (the
    rule for that case: draw from p at that position). At position 0 of
    every sequence the target logit of the drafted token is -inf (p(x) = 0,
    always rejected) and the draft row equals the target row everywhere else,
    with a finite -50 at the drafted token: q(x) is about 1e-37, the two
    normalisers are the same in fp64 (the oracle) and in the kernels' fp32
    sums, so both see a residual of exactly zero and draw from p_0 with the
    sampling uniform. The c2 shape, so the kernels take their one-workgroup
    fallback that re-reads the row; its time is printed next to a plain call."""
    cfg = CHAIN_CONFIGS["c2"]
    inp = chain_inputs(cfg, device="cuda")
    _say("vanished residual", cfg.name, "row 0: target -inf and draft -50 at the drafted token")
    B = cfg.B
    bi = torch.arange(B, device="cuda")
    x0 = inp["draft_tokens"][:, 0].long()
    target = inp["target"].clone()
    draft = inp["draft"].clone()
    draft[:, 0, :] = target[:, 0, :]
    target[bi, 0, x0] = float("-inf")
    draft[bi, 0, x0] = -50.0
    case = {**inp, "target": target, "draft": draft}
    plain = _run(sv, inp)
    out = _run(sv, case)
    check_chain_structure(out, cfg.K, cfg.V)
    assert int(out["err_flags"].item()) == 0
    ref = oracle_chain(case)
    assert np.all(ref["accept_len"] == 0) and np.all(ref["residual_mass"] == 0.0)
    assert np.all(to_np_i(out["accept_len"]) == 0)
    assert np.all(out["residual_mass"].cpu().numpy() == 0.0)
    assert np.all(out["p_draft"][:, 0].cpu().numpy() == 0.0)
    rep = compare_chain(out, ref)
    print("vanished residual", rep, flush=True)
    assert_chain_parity(rep)
    # the drawn tokens follow p_0 (they are p_0's inverse CDF at u_K): never the drafted token
    assert np.all(to_np_i(out["out_tokens"])[:, 0] != to_np_i(x0))
    # time of the fallback against the plain call on the same shape
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for _ in range(5):
        sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"], inp["uniforms"])
    ev[1].record()
    ev[2].record()
    for _ in range(5):
        sv.sv_verify_chain(case["target"], case["draft"], case["draft_tokens"], case["temperature"], case["uniforms"])
    ev[3].record()
    torch.cuda.synchronize()
    print(f"vanished residual: {ev[2].elapsed_time(ev[3]) / 5 * 1e3:.1f} us per call against "
          f"{ev[0].elapsed_time(ev[1]) / 5 * 1e3:.1f} us for the plain call", flush=True)
    del plain
