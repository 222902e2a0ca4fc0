"""GPU parity of the per-position entropy that sv_verify_chain emits from its
statistics pass, against the oracle's -sum p ln p in float64.

Bar: |H_gpu - H| <= 1e-5 * H + 2e-6 nats on every valid row (fp32 per-thread
sums on bf16 / fp32 inputs; the absolute floor covers near point masses, where
H is the difference of two small terms of fp32 rounding). Asking for the
entropy must leave every other output bit-identical. Every case prints its
name, shape and seed before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import record_parity, oracle_chain, to_np64
from workloads import CHAIN_CONFIGS, chain_inputs

pytestmark = pytest.mark.gpu

H_REL, H_ABS = 1e-5, 2e-6


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "these tests need a GPU"
    import rejection_sampling_verification_sv_amd as m
    m.library()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _call(sv, inp, **kw):
    out = sv.sv_verify_chain(inp["target"], inp["draft"], inp["draft_tokens"], inp["temperature"],
                             inp["uniforms"], **kw)
    torch.cuda.synchronize()
    return out


def _check(sv, inp, rows=None, label="", record=False):
    """Entropy against the oracle (on `rows`, default all) and the other outputs
    against a call without the entropy; returns (max abs err, max rel err)."""
    plain = _call(sv, inp)
    withh = _call(sv, inp, want_entropy=True)
    for k in ("accept_len", "out_tokens", "p_draft", "q_draft", "residual_mass", "err_flags"):
        assert torch.equal(plain[k], withh[k]), f"{label}: {k} changed when the entropy was requested"
    if rows is None and inp["target"].shape[0] > 16:  # fp64 copies of a few sequences at a time
        parts = [oracle_chain(inp, np.arange(s0, min(inp["target"].shape[0], s0 + 16)), with_entropy=True)
                 for s0 in range(0, inp["target"].shape[0], 16)]
        ref = {k: np.concatenate([p_[k] for p_ in parts]) for k in ("entropy", "valid")}
    else:
        ref = oracle_chain(inp, rows, with_entropy=True)
    h = to_np64(withh["entropy"] if rows is None else withh["entropy"][rows.cuda() if torch.is_tensor(rows) else rows])
    valid = ref["valid"]
    err = np.abs(h[valid] - ref["entropy"][valid])
    bound = H_REL * ref["entropy"][valid] + H_ABS
    assert np.all(err <= bound), f"{label}: worst excess {np.max(err - bound)} (max err {err.max()})"
    rel = err / np.maximum(ref["entropy"][valid], 1e-12)
    print(label, "rows", valid.sum(), "max abs err %.3g" % err.max(initial=0), "max rel err %.3g" % rel.max(initial=0),
          flush=True)
    if record:
        record_parity(label, call="sv_verify_chain (entropy)", distributions=int(valid.sum() * h.shape[1]),
                      max_abs_err_nats=float(err.max(initial=0.0)), max_rel_err=float(rel.max(initial=0.0)),
                      bar="|H - H_oracle| <= 1e-5 H + 2e-6 nats")
    return err.max(initial=0.0), rel.max(initial=0.0)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_entropy_of_the_chain_workloads(sv, name):
    cfg = CHAIN_CONFIGS[name]
    _say("entropy", cfg.name)
    inp = chain_inputs(cfg, device="cuda")
    if name == "c2":  # the one-launch form, with its entropy variant
        B, _, V = inp["target"].shape
        assert sv.sv_chain_form(B, inp["draft"].shape[1], V, inp["target"].dtype, True, True) == 2
    _check(sv, inp, label=cfg.name, record=True)


def test_entropy_c3_per_row_temperature_full(sv):
    cfg = CHAIN_CONFIGS["c3_s1.0"]
    _say("entropy", cfg.name, "all 256 sequences")
    inp = chain_inputs(cfg, device="cuda")
    _check(sv, inp, label=cfg.name, record=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,K,V,offset", [(5, 3, 1000, 0), (4, 2, 4099, 1), (3, 0, 128256, 0), (2, 4, 33, 0)])
def test_entropy_shapes_and_layouts(sv, B, K, V, offset, dtype):
    # offset 1 puts every row off the 16-byte grid (the segments layout)
    _say("entropy shapes B", B, "K", K, "V", V, "offset", offset, dtype, "Philox seed", 40 + V)
    rng = np.random.Generator(np.random.Philox(40 + V))
    n_t, n_d = B * (K + 1) * V, B * K * V
    flat_t = torch.from_numpy(rng.normal(0, 3, n_t + offset).astype(np.float32)).to(dtype)
    flat_d = torch.from_numpy(rng.normal(0, 3, max(n_d, 1) + offset).astype(np.float32)).to(dtype)
    target = flat_t.cuda()[offset:offset + n_t].view(B, K + 1, V)
    draft = flat_d.cuda()[offset:offset + n_d].view(B, K, V) if K else None
    inp = {"target": target, "draft": draft,
           "draft_tokens": torch.from_numpy(rng.integers(0, V, (B, K)).astype(np.int32)).cuda() if K else None,
           "temperature": torch.from_numpy(rng.uniform(0.4, 1.4, B).astype(np.float32)).cuda(),
           "uniforms": torch.from_numpy(rng.random((B, K + 1), dtype=np.float32)).cuda()}
    _check(sv, inp, label=f"B{B} K{K} V{V} off{offset}")


def test_entropy_with_masked_tokens_and_bad_rows(sv):
    _say("entropy: -inf logits, a near point mass, an invalid temperature")
    rng = np.random.Generator(np.random.Philox(41))
    B, K, V = 4, 2, 3000
    t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 1, (B, K, V))).astype(np.float32)
    t[0, :, ::2] = -np.inf      # half the vocabulary masked
    t[1, 0, 5] = 60.0           # a near point mass at T = 0.5
    T = np.array([1.0, 0.5, 0.0, 1.3], np.float32)  # row 2: invalid
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[0] = 1                    # drafted tokens with p > 0 in row 0
    inp = {"target": torch.from_numpy(t).cuda(), "draft": torch.from_numpy(d).cuda(),
           "draft_tokens": torch.from_numpy(x).cuda(), "temperature": torch.from_numpy(T).cuda(),
           "uniforms": torch.from_numpy(rng.random((B, K + 1), dtype=np.float32)).cuda()}
    out = _call(sv, inp, want_entropy=True)
    h = to_np64(out["entropy"])
    assert np.all(np.isnan(h[2])), "an invalid temperature gives NaN entropy"
    keep = [0, 1, 3]
    sub = {k: (v[keep] if torch.is_tensor(v) else v) for k, v in inp.items()}
    ref = oracle_chain(sub, with_entropy=True)
    err = np.abs(h[keep] - ref["entropy"])
    assert np.all(err <= H_REL * ref["entropy"] + H_ABS), err.max()
    assert h[1, 0] < 1e-3 and np.all((h >= -H_ABS) | np.isnan(h))
