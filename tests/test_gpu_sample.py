"""GPU parity of sv_sample_rows (draft-side sampling) against the CPU oracle.

Bar: drawn tokens bit-exact, except rows whose uniform lies within 1e-6 of a
CDF boundary of the oracle's drawn token (counted, never hidden); q of the
drawn token within 1e-5 relative. Every case prints its name, shape and seed
before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import REL_TOL, record_parity, to_np64, to_np_i
from workloads import CHAIN_CONFIGS, sample_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _expected_flagged(logits, temperature):
    """Expected number of near-boundary rows: a uniform falls within the flag
    window of one of the drawn token's two CDF boundaries with probability
    sum_v min(q(v), 2 * FLAG_WINDOW) (rows of flat distributions flag often)."""
    T = np.ones(logits.shape[0]) if temperature is None else to_np64(temperature)
    total = 0.0
    for r0 in range(0, logits.shape[0], 64):
        q = oracle.temperature_softmax(to_np64(logits[r0:r0 + 64]), T[r0:r0 + 64])
        total += float(np.minimum(q, 2 * oracle.FLAG_WINDOW).sum())
    return total


def _oracle_rows(logits, temperature, uniforms, per=256):
    """The oracle's draft-side sampling, `per` rows at a time."""
    parts = []
    for r0 in range(0, logits.shape[0], per):
        r1 = min(logits.shape[0], r0 + per)
        parts.append(oracle.sample_rows(to_np64(logits[r0:r1]),
                                        None if temperature is None else to_np64(temperature[r0:r1]),
                                        to_np64(uniforms[r0:r1])))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def _compare(out, logits, temperature, uniforms, record=None):
    """Tokens exact outside the flag window, q(token) to REL_TOL; returns (rows, flagged)."""
    t_ref, p_ref, lo, hi = _oracle_rows(logits, temperature, uniforms)
    u = to_np64(uniforms)
    flagged = (np.abs(u - lo) < oracle.FLAG_WINDOW) | (np.abs(hi - u) < oracle.FLAG_WINDOW)
    tok = to_np_i(out["tokens"])
    bad = (tok != t_ref) & ~flagged
    assert not bad.any(), f"{bad.sum()} unflagged token mismatches, first rows {np.nonzero(bad)[0][:8]}"
    same = tok == t_ref
    prob = to_np64(out["prob"])
    rel = np.abs(prob[same] - p_ref[same]) / np.maximum(p_ref[same], 1e-30)
    assert rel.max(initial=0.0) <= REL_TOL, f"max relative error of q(token) {rel.max()}"
    expected = _expected_flagged(logits, temperature)
    if record is not None:
        margin = np.minimum(u - lo, hi - u)
        record_parity(record, call="sv_sample_rows", rows=len(u), flagged=int(flagged.sum()),
                      expected_flagged=expected, mismatched_unflagged=int(bad.sum()),
                      mismatched_flagged=int((~same & flagged).sum()), max_rel_prob=float(rel.max(initial=0.0)),
                      min_margin=float(margin.min()))
    assert flagged.sum() <= 3 * expected + 3, f"{flagged.sum()} flagged rows, about {expected:.1f} expected"
    assert np.all((tok >= 0) & (tok < logits.shape[1]))
    return len(u), int(flagged.sum())


def _run(sv, inp, **kw):
    out = sv.sv_sample_rows(inp["logits"], inp["temperature"], inp["uniforms"], **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_draft_rows_of_the_chain_workloads(sv, name):
    cfg = CHAIN_CONFIGS[name]
    _say("sample rows of", cfg.name, "B*K =", cfg.B * cfg.K, "V =", cfg.V, "seed stream 6")
    inp = sample_inputs(cfg, device="cuda")
    out = _run(sv, inp)
    assert int(out["err_flags"].item()) == 0
    rows, flagged = _compare(out, inp["logits"], inp["temperature"], inp["uniforms"],
                             record=f"sample_rows_of_{cfg.name}")
    print(name, "rows", rows, "flagged", flagged, flush=True)


def test_c3_draft_rows_full(sv):
    # all 2048 rows of V = 152064 with per-row temperatures U[0.3, 1.3]
    cfg = CHAIN_CONFIGS["c3_s1.0"]
    _say("sample rows of", cfg.name, "B*K =", cfg.B * cfg.K, "V =", cfg.V)
    inp = sample_inputs(cfg, device="cuda")
    out = _run(sv, inp)
    assert int(out["err_flags"].item()) == 0
    rows, flagged = _compare(out, inp["logits"], inp["temperature"], inp["uniforms"],
                             record=f"sample_rows_of_{cfg.name}")
    assert rows == cfg.B * cfg.K
    print(cfg.name, "rows", rows, "flagged", flagged, flush=True)


def test_law_of_the_drawn_token(sv):
    # 10^6 rows of one 16-token distribution: the drawn tokens follow q
    from scipy import stats
    _say("law: 1e6 rows, V = 16, f32, T = 0.8, Philox seed 21")
    rng = np.random.Generator(np.random.Philox(21))
    V, n, T = 16, 1_000_000, 0.8
    row = rng.normal(0.0, 2.0, V).astype(np.float32)
    logits = torch.from_numpy(np.broadcast_to(row, (n, V)).copy()).cuda()
    u = torch.from_numpy(rng.random(n, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": torch.full((n,), T, device="cuda"), "uniforms": u})
    q = np.exp(row.astype(np.float64) / T - (row / T).max())
    q /= q.sum()
    counts = np.bincount(to_np_i(out["tokens"]), minlength=V)
    assert stats.chisquare(counts, q * n).pvalue > 0.01


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 16, 33, 1000, 2048, 2049, 5000])
def test_edge_shapes(sv, V, dtype):
    _say("edge", "R = 37", "V =", V, dtype, "Philox seed", 1000 + V)
    rng = np.random.Generator(np.random.Philox(1000 + V))
    R = 37
    logits = torch.from_numpy(rng.normal(0, 2.5, (R, V)).astype(np.float32)).to(dtype).cuda()
    T = torch.from_numpy(rng.uniform(0.3, 1.5, R).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": T, "uniforms": u})
    assert int(out["err_flags"].item()) == 0
    _compare(out, logits, T, u)


def test_unaligned_rows(sv):
    # a row base off the 16-byte grid takes the segments layout
    _say("unaligned rows: bf16 V = 4099 viewed at offset 1")
    rng = np.random.Generator(np.random.Philox(31))
    R, V = 24, 4099
    flat = torch.from_numpy(rng.normal(0, 2, R * V + 1).astype(np.float32)).to(torch.bfloat16).cuda()
    logits = flat[1:].view(R, V)
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": None, "uniforms": u})
    assert int(out["err_flags"].item()) == 0
    _compare(out, logits, None, u)


def test_empty_and_default_temperature(sv):
    _say("R = 0; and T = NULL against T = 1")
    out = _run(sv, {"logits": torch.zeros((0, 100), device="cuda"), "temperature": None,
                    "uniforms": torch.zeros((0,), device="cuda")})
    assert out["tokens"].numel() == 0
    rng = np.random.Generator(np.random.Philox(32))
    logits = torch.from_numpy(rng.normal(0, 2, (50, 3000)).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.random(50, dtype=np.float32)).cuda()
    a = _run(sv, {"logits": logits, "temperature": None, "uniforms": u})
    b = _run(sv, {"logits": logits, "temperature": torch.ones(50, device="cuda"), "uniforms": u})
    assert torch.equal(a["tokens"], b["tokens"]) and torch.equal(a["prob"], b["prob"])


def test_data_errors_are_flagged_per_row(sv):
    _say("bad temperatures and a NaN logit in some rows")
    rng = np.random.Generator(np.random.Philox(33))
    R, V = 8, 1000
    logits = torch.from_numpy(rng.normal(0, 2, (R, V)).astype(np.float32))
    T = torch.ones(R)
    T[1] = 0.0
    T[2] = float("nan")
    logits[4, 17] = float("nan")
    logits, T = logits.cuda(), T.cuda()
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": T, "uniforms": u})
    tok = to_np_i(out["tokens"])
    prob = to_np64(out["prob"])
    flags = int(out["err_flags"].item())
    assert flags & sv.SV_ERRF_TEMPERATURE and flags & sv.SV_ERRF_NONFINITE
    for r in (1, 2, 4):
        assert tok[r] == -1 and np.isnan(prob[r])
    good = [r for r in range(R) if r not in (1, 2, 4)]
    _compare({"tokens": out["tokens"][good], "prob": out["prob"][good]}, logits[good], T[good], u[good])


def test_repeat_is_bit_identical(sv):
    _say("repeat: c2 draft rows twice")
    inp = sample_inputs(CHAIN_CONFIGS["c2"], device="cuda")
    a = _run(sv, inp)
    b = _run(sv, inp)
    assert torch.equal(a["tokens"], b["tokens"]) and torch.equal(a["prob"], b["prob"])


@pytest.mark.parametrize("dtype,V,R", [(torch.bfloat16, 8, 5000), (torch.bfloat16, 2048, 2049),
                                       (torch.float32, 4, 3000), (torch.bfloat16, 12288, 700)])
def test_many_short_rows(sv, dtype, V, R):
    # units of the stream much shorter than a wave's share: waves cross rows
    # (each row its own scale), take several units each, or none at all
    # (more waves than units), and every group's counter still closes
    _say("many short rows: R =", R, "V =", V, dtype, "Philox seed", 50 + V)
    rng = np.random.Generator(np.random.Philox(50 + V))
    logits = torch.from_numpy(rng.normal(0, 2.5, (R, V)).astype(np.float32)).to(dtype).cuda()
    T = torch.from_numpy(rng.uniform(0.3, 1.5, R).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": T, "uniforms": u})
    assert int(out["err_flags"].item()) == 0
    _compare(out, logits, T, u)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 600000), (torch.float32, 300000)])
def test_long_rows_reread_records(sv, dtype, V):
    # more than 128 records (256-vector segments) per row: the draw re-reads its records
    _say("long rows: R = 5, V =", V, dtype, "Philox seed 34")
    rng = np.random.Generator(np.random.Philox(34))
    R = 5
    logits = torch.from_numpy(rng.normal(0, 3, (R, V)).astype(np.float32)).to(dtype).cuda()
    T = torch.from_numpy(rng.uniform(0.5, 1.5, R).astype(np.float32)).cuda()
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).cuda()
    out = _run(sv, {"logits": logits, "temperature": T, "uniforms": u})
    assert int(out["err_flags"].item()) == 0
    _compare(out, logits, T, u)
