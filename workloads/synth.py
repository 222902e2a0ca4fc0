"""Seeded synthetic workloads shaped like the pages' speculative-decoding traffic.

What is drawn, per configuration (all seeded, nothing read from disk):

* chain verification: target logits ``[B, K+1, V]`` = N(0, sigma_t^2) plus an
  optional Zipf log-prior ``-s * ln(v + 1)``; draft logits ``[B, K, V]`` =
  target + N(0, sigma_d^2) drawn in float64 (or float32 on a GPU) and rounded
  to the storage dtype independently of the target; draft tokens drawn from the
  draft distribution at the row's temperature with the Gumbel-max trick on the
  *stored* draft logits; one temperature per sequence; uniforms ``[B, K+1]`` in
  [0, 1) (columns ``0..K-1`` for the accept tests, column ``K`` for the
  replacement / bonus draw).
* greedy tree verification: a candidate tree given as a parent array (see
  :func:`tree_parents_ranked`), target logits ``[B, N+1, V]``, and node tokens
  taken as the parent position's r-th highest target logit (r = the node's rank
  among its siblings) with a fixed chance of being replaced by a uniform id.

Random streams. On the CPU every stream is
``numpy.random.Generator(Philox(SeedSequence([SEED_BASE, config_id, variant,
stream, iteration])))``. On a GPU device the same SeedSequence seeds a
``torch.Generator`` on that device (Philox4x32-10 in PyTorch's ROCm build), so a
CPU draw and a GPU draw of the same configuration are different (equally valid)
samples. Stream ids: 0 target logits, 1 draft noise, 2 draft-token Gumbel
noise, 3 uniforms, 4 temperatures, 5 tree token replacement, 6 uniforms of
the draft-side sampling workload.

* draft-side sampling: the draft logits of a chain configuration taken as
  ``B * K`` independent rows ``[B*K, V]``, each with its sequence's
  temperature and one uniform in [0, 1).

Gumbel-max (argmax of logits/T + Gumbel noise) is how the *drafter* side draws
its proposals; it belongs to input generation, not to the verification step,
and no softmax is formed here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

SEED_BASE = 20261202

STREAM_TARGET = 0
STREAM_DRAFT_NOISE = 1
STREAM_DRAFT_TOKENS = 2
STREAM_UNIFORMS = 3
STREAM_TEMPERATURE = 4
STREAM_TREE_REPLACE = 5
STREAM_SAMPLE_UNIFORMS = 6
STREAM_HIDDEN = 7
STREAM_WEIGHT = 8
STREAM_DRAFT_WEIGHT = 9

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class ChainConfig:
    """One chain-verification workload (B sequences, K drafted tokens, vocab V)."""

    name: str
    config_id: int
    B: int
    K: int
    V: int
    dtype: str  # "f32" or "bf16": storage dtype of both logit tensors
    target_sigma: float
    zipf_s: float  # 0.0 = no log-prior
    draft_sigma: float
    temperature: Optional[float] = 1.0  # one temperature for every sequence ...
    temperature_range: Optional[Tuple[float, float]] = None  # ... or U[lo, hi] per sequence
    variant: int = 0
    iterations: int = 1  # back-to-back calls, fresh uniforms for each

    @property
    def rows(self) -> int:
        return self.B * (2 * self.K + 1)

    @property
    def elements(self) -> int:
        """Logit elements one verification call consumes (rows x vocab)."""
        return self.rows * self.V

    @property
    def logit_bytes(self) -> int:
        return self.elements * (4 if self.dtype == "f32" else 2)

    def with_(self, **kw) -> "ChainConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class TreeConfig:
    """One greedy tree-verification workload (B sequences, N tree nodes)."""

    name: str
    config_id: int
    B: int
    N: int
    V: int
    dtype: str
    target_sigma: float
    branching: Tuple[int, ...]
    replace_prob: float
    variant: int = 0

    @property
    def rows(self) -> int:
        return self.B * (self.N + 1)

    @property
    def elements(self) -> int:
        return self.rows * self.V

    @property
    def logit_bytes(self) -> int:
        return self.elements * (4 if self.dtype == "f32" else 2)

    def with_(self, **kw) -> "TreeConfig":
        return dataclasses.replace(self, **kw)


CHAIN_CONFIGS = {
    "c1": ChainConfig("chain_b4_k4_v32000_f32", 1, 4, 4, 32000, "f32", 3.0, 0.0, 1.0, 1.0),
    "c2": ChainConfig("chain_b64_k5_v128256_bf16", 2, 64, 5, 128256, "bf16", 2.5, 1.1, 0.8, 0.7),
    "c3_s0.3": ChainConfig("chain_b256_k8_v152064_bf16_sigma0.3", 3, 256, 8, 152064, "bf16",
                           3.0, 0.0, 0.3, None, (0.3, 1.3), variant=0),
    "c3_s1.0": ChainConfig("chain_b256_k8_v152064_bf16_sigma1.0", 3, 256, 8, 152064, "bf16",
                           3.0, 0.0, 1.0, None, (0.3, 1.3), variant=1),
    "c3_s3.0": ChainConfig("chain_b256_k8_v152064_bf16_sigma3.0", 3, 256, 8, 152064, "bf16",
                           3.0, 0.0, 3.0, None, (0.3, 1.3), variant=2),
    "c5": ChainConfig("chain_b1024_k6_v256000_bf16_x10", 5, 1024, 6, 256000, "bf16",
                      3.0, 1.0, 1.5, 1.0, iterations=10),
}

# Monte Carlo losslessness workload: tiny vocabulary, the same logits for every
# trial, a fresh draft draw and fresh uniforms per trial.
MC_CONFIG = ChainConfig("chain_mc_v16_k3_f32", 1, 1_000_000, 3, 16, "f32", 3.0, 0.0, 1.0, 1.0,
                        variant=1)

TREE_CONFIGS = {
    "c4": TreeConfig("tree_b32_n64_v128256_bf16", 4, 32, 64, 128256, "bf16", 3.0,
                     (4, 3, 2, 2, 1), 0.3),
}


@dataclasses.dataclass(frozen=True)
class SampleTreeConfig:
    """One sampling tree-verification workload: the candidate tree of a greedy
    configuration, draft logits at every position, node tokens drawn from the
    draft distribution at their parent's position (siblings independently)."""

    name: str
    config_id: int
    B: int
    N: int
    V: int
    dtype: str
    target_sigma: float
    draft_sigma: float
    temperature: float
    branching: Tuple[int, ...]
    variant: int = 0

    @property
    def rows(self) -> int:
        return 2 * self.B * (self.N + 1)

    @property
    def elements(self) -> int:
        return self.rows * self.V

    @property
    def logit_bytes(self) -> int:
        return self.elements * (4 if self.dtype == "f32" else 2)

    def with_(self, **kw) -> "SampleTreeConfig":
        return dataclasses.replace(self, **kw)


SAMPLE_TREE_CONFIGS = {
    "c4s": SampleTreeConfig("tree_sampling_b32_n64_v128256_bf16", 6, 32, 64, 128256, "bf16", 3.0, 1.0, 1.0,
                            (4, 3, 2, 2, 1)),
}


@dataclasses.dataclass(frozen=True)
class LMHeadConfig:
    """Chain verification whose target logits come out of the target's LM
    head: hidden states ``[B, K+1, H]`` and head weights ``[V, H]`` (bf16).

    The hidden states are N(0, 1) with a last column of ones; the weights are
    N(0, target_sigma^2 / (H - 1)) with a last column holding the Zipf
    log-prior -s ln(v + 1), so the logits look like the chain workload's
    N(0, target_sigma^2) + prior. The draft's logits come from its own head:
    the same hidden states through the weights plus N(0, draft_sigma^2 /
    (H - 1)) noise, so draft - target has about draft_sigma's spread.
    ``exact``: integer hidden states and weights in [-3, 3] (draft head:
    each weight moved by +-1 with probability 0.2 each), whose sums a float32
    accumulation forms exactly; the temperature then scales those integer
    logits to the same spread.
    """

    name: str
    config_id: int
    B: int
    K: int
    V: int
    H: int
    target_sigma: float
    zipf_s: float
    draft_sigma: float
    temperature: float
    exact: bool = False
    variant: int = 0

    @property
    def rows(self) -> int:
        return self.B * (2 * self.K + 1)

    def with_(self, **kw) -> "LMHeadConfig":
        return dataclasses.replace(self, **kw)


LM_HEAD_CONFIGS = {
    "c2h": LMHeadConfig("lm_head_chain_b64_k5_v128256_h8192_bf16", 7, 64, 5, 128256, 8192, 2.5, 1.1, 0.8, 0.7),
    "c2h_int": LMHeadConfig("lm_head_chain_b64_k5_v128256_h8192_bf16_integer", 8, 64, 5, 128256, 8192, 2.5, 1.1,
                            0.8, 0.7, exact=True),
}


# ----------------------------------------------------------------------------- seeds

def _seed_sequence(config_id: int, variant: int, stream: int, iteration: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_BASE, int(config_id), int(variant), int(stream), int(iteration)])


def seed_stream(config_id: int, variant: int, stream: int, iteration: int = 0) -> np.random.Generator:
    """The numpy Philox generator for one (configuration, stream, iteration)."""
    return np.random.Generator(np.random.Philox(_seed_sequence(config_id, variant, stream, iteration)))


def _torch_generator(device, config_id: int, variant: int, stream: int, iteration: int = 0) -> torch.Generator:
    state = _seed_sequence(config_id, variant, stream, iteration).generate_state(1, np.uint64)[0]
    g = torch.Generator(device=device)
    g.manual_seed(int(state) & ((1 << 63) - 1))
    return g


def _is_cpu(device) -> bool:
    return torch.device(device).type == "cpu"


def zipf_log_prior(V: int, s: float) -> np.ndarray:
    """Log-prior ``-s * ln(rank)`` with rank = token id + 1 (float64, length V)."""
    return -float(s) * np.log(np.arange(1, V + 1, dtype=np.float64))


# ----------------------------------------------------------------------------- draft tokens

def sample_draft_tokens_gumbel(draft_logits: torch.Tensor, temperature: torch.Tensor,
                               generator, chunk_rows: int = 1 << 12) -> torch.Tensor:
    """Draw one token per draft row, x ~ softmax(logits / T), by the Gumbel-max trick.

    ``draft_logits`` is ``[B, K, V]`` (any float dtype; its stored values are
    used), ``temperature`` is ``[B]``. ``generator`` is a numpy Generator on
    the CPU path (noise in float64) or a torch Generator on the device path
    (noise in float32). Returns int32 ``[B, K]`` on the logits' device.
    """
    B, K, V = draft_logits.shape
    out = torch.empty((B, K), dtype=torch.int32, device=draft_logits.device)
    if B == 0 or K == 0:
        return out
    per_seq = max(1, chunk_rows // max(K, 1))
    for b0 in range(0, B, per_seq):
        b1 = min(B, b0 + per_seq)
        if isinstance(generator, np.random.Generator):
            d = draft_logits[b0:b1].to(torch.float64).numpy()
            T = temperature[b0:b1].to(torch.float64).numpy()[:, None, None]
            g = generator.gumbel(size=d.shape)
            out[b0:b1] = torch.from_numpy(np.argmax(d / T + g, axis=-1).astype(np.int32))
        else:
            d = draft_logits[b0:b1].to(torch.float32)
            T = temperature[b0:b1].to(torch.float32)[:, None, None]
            u = torch.rand(d.shape, generator=generator, device=d.device, dtype=torch.float32)
            u = u.clamp_(min=torch.finfo(torch.float32).tiny)
            g = -torch.log(-torch.log(u))
            out[b0:b1] = torch.argmax(d / T + g, dim=-1).to(torch.int32)
    return out


# ----------------------------------------------------------------------------- chain inputs

def chain_temperatures(cfg: ChainConfig, device="cpu") -> torch.Tensor:
    if cfg.temperature_range is None:
        return torch.full((cfg.B,), float(cfg.temperature), dtype=torch.float32, device=device)
    lo, hi = cfg.temperature_range
    g = seed_stream(cfg.config_id, cfg.variant, STREAM_TEMPERATURE)
    t = g.uniform(lo, hi, size=cfg.B).astype(np.float32)
    return torch.from_numpy(t).to(device)


def chain_uniforms(cfg: ChainConfig, iteration: int = 0, device="cpu") -> torch.Tensor:
    """Uniforms in [0, 1), float32 ``[B, K+1]`` for one verification call."""
    shape = (cfg.B, cfg.K + 1)
    if _is_cpu(device):
        g = seed_stream(cfg.config_id, cfg.variant, STREAM_UNIFORMS, iteration)
        return torch.from_numpy(g.random(shape, dtype=np.float32))
    g = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_UNIFORMS, iteration)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def _chain_logits_cpu(cfg: ChainConfig):
    B, K, V = cfg.B, cfg.K, cfg.V
    dt = _TORCH_DTYPES[cfg.dtype]
    prior = zipf_log_prior(V, cfg.zipf_s) if cfg.zipf_s else None
    gt = seed_stream(cfg.config_id, cfg.variant, STREAM_TARGET)
    gd = seed_stream(cfg.config_id, cfg.variant, STREAM_DRAFT_NOISE)
    target = torch.empty((B, K + 1, V), dtype=dt)
    draft = torch.empty((B, K, V), dtype=dt)
    for b in range(B):  # one sequence at a time keeps float64 temporaries small
        t64 = gt.standard_normal((K + 1, V)) * cfg.target_sigma
        if prior is not None:
            t64 += prior
        d64 = t64[:K] + gd.standard_normal((K, V)) * cfg.draft_sigma
        target[b] = torch.from_numpy(t64).to(dt)
        draft[b] = torch.from_numpy(d64).to(dt)
    return target, draft


def _chain_logits_device(cfg: ChainConfig, device):
    B, K, V = cfg.B, cfg.K, cfg.V
    dt = _TORCH_DTYPES[cfg.dtype]
    gt = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_TARGET)
    gd = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_NOISE)
    prior = None
    if cfg.zipf_s:
        prior = torch.from_numpy(zipf_log_prior(V, cfg.zipf_s)).to(device=device, dtype=torch.float32)
    target = torch.empty((B, K + 1, V), dtype=dt, device=device)
    draft = torch.empty((B, K, V), dtype=dt, device=device)
    per = max(1, (1 << 27) // max(1, (K + 1) * V))  # sequences per chunk: bounded float32 temporaries
    for b0 in range(0, B, per):
        b1 = min(B, b0 + per)
        t32 = torch.randn((b1 - b0, K + 1, V), generator=gt, device=device) * cfg.target_sigma
        if prior is not None:
            t32 += prior
        d32 = t32[:, :K] + torch.randn((b1 - b0, K, V), generator=gd, device=device) * cfg.draft_sigma
        target[b0:b1] = t32.to(dt)
        draft[b0:b1] = d32.to(dt)
        del t32, d32
    return target, draft


def chain_inputs(cfg: ChainConfig, device="cpu", iteration: int = 0) -> dict:
    """All inputs of one chain-verification call, as torch tensors on ``device``.

    Keys: ``target [B,K+1,V]``, ``draft [B,K,V]`` (cfg.dtype), ``draft_tokens
    [B,K]`` int32, ``temperature [B]`` float32, ``uniforms [B,K+1]`` float32.
    Logits and tokens do not depend on ``iteration``; uniforms do.
    """
    temperature = chain_temperatures(cfg, device)
    if _is_cpu(device):
        target, draft = _chain_logits_cpu(cfg)
        gx = seed_stream(cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
    else:
        target, draft = _chain_logits_device(cfg, device)
        gx = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
    tokens = sample_draft_tokens_gumbel(draft, temperature, gx)
    return {
        "target": target,
        "draft": draft,
        "draft_tokens": tokens,
        "temperature": temperature,
        "uniforms": chain_uniforms(cfg, iteration, device),
    }


def sample_inputs(cfg: ChainConfig, device="cpu", iteration: int = 0) -> dict:
    """Inputs of one draft-side sampling call built from a chain configuration.

    Keys: ``logits [B*K, V]`` (the configuration's draft logits, one row per
    drafted position), ``temperature [B*K]`` float32 (each sequence's
    temperature repeated over its positions) and ``uniforms [B*K]`` float32 in
    [0, 1) from stream 6. The logits do not depend on ``iteration``; the
    uniforms do.
    """
    if cfg.K < 1:
        raise ValueError("draft-side sampling needs K >= 1 drafted positions")
    if _is_cpu(device):
        _, draft = _chain_logits_cpu(cfg)
    else:
        _, draft = _chain_logits_device(cfg, device)
    rows = cfg.B * cfg.K
    temperature = chain_temperatures(cfg, device).repeat_interleave(cfg.K)
    if _is_cpu(device):
        g = seed_stream(cfg.config_id, cfg.variant, STREAM_SAMPLE_UNIFORMS, iteration)
        u = torch.from_numpy(g.random(rows, dtype=np.float32))
    else:
        g = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_SAMPLE_UNIFORMS, iteration)
        u = torch.rand((rows,), generator=g, device=device, dtype=torch.float32)
    return {"logits": draft.reshape(rows, cfg.V), "temperature": temperature, "uniforms": u}


def mc_chain_inputs(cfg: ChainConfig = MC_CONFIG, trials: Optional[int] = None) -> dict:
    """Monte Carlo workload on the CPU: one fixed (target, draft) logit set.

    Returns ``target_row [K+1,V]`` and ``draft_row [K,V]`` (stored dtype), plus
    per-trial ``draft_tokens [n,K]`` (x_k ~ q_k, Gumbel-max in float64 on the
    stored draft logits), ``uniforms [n,K+1]`` and ``temperature [n]``.
    """
    n = cfg.B if trials is None else int(trials)
    one = cfg.with_(B=1)
    target, draft = _chain_logits_cpu(one)
    temperature = torch.full((n,), float(cfg.temperature), dtype=torch.float32)
    gx = seed_stream(cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
    tokens = sample_draft_tokens_gumbel(draft.expand(n, cfg.K, cfg.V), temperature, gx, chunk_rows=1 << 18)
    gu = seed_stream(cfg.config_id, cfg.variant, STREAM_UNIFORMS)
    uniforms = torch.from_numpy(gu.random((n, cfg.K + 1), dtype=np.float32))
    return {
        "target_row": target[0],
        "draft_row": draft[0],
        "draft_tokens": tokens,
        "temperature": temperature,
        "uniforms": uniforms,
    }


# ----------------------------------------------------------------------------- trees

def tree_parents_ranked(branching: Sequence[int], n_nodes: int):
    """A candidate tree of ``n_nodes`` nodes cut from the full tree of ``branching``.

    The full tree has ``branching[d]`` children under every node at depth ``d``
    (the root, the last accepted token, is depth 0). Each node is named by its
    rank path ``(r_1, .., r_d)`` (r_i = rank among siblings, 0 = the parent's
    most likely continuation). Nodes are ordered by (sum of ranks, depth, rank
    path) and the first ``n_nodes`` kept; a parent always sorts before its
    children, so every prefix of this order is a valid tree and the order is
    topological. Returns ``(parents, ranks)``: int32 arrays of length
    ``n_nodes``, ``parents[i]`` = -1 for a child of the root, else the parent's
    index (< i); ``ranks[i]`` = the node's own sibling rank r_d.
    """
    paths = []

    def walk(prefix):
        d = len(prefix)
        if d == len(branching):
            return
        for r in range(branching[d]):
            p = prefix + (r,)
            paths.append(p)
            walk(p)

    walk(())
    paths.sort(key=lambda p: (sum(p), len(p), p))
    if n_nodes > len(paths):
        raise ValueError(f"the full tree has only {len(paths)} nodes")
    kept = paths[:n_nodes]
    index = {p: i for i, p in enumerate(kept)}
    parents = np.array([-1 if len(p) == 1 else index[p[:-1]] for p in kept], dtype=np.int32)
    ranks = np.array([p[-1] for p in kept], dtype=np.int32)
    return parents, ranks


def tree_inputs(cfg: TreeConfig, device="cpu") -> dict:
    """Inputs of one greedy tree-verification call on ``device``.

    Keys: ``target [B,N+1,V]`` (position 0 = the root, position i+1 = node i),
    ``node_tokens [B,N]`` int32, ``parents [N]`` int32.
    """
    B, N, V = cfg.B, cfg.N, cfg.V
    dt = _TORCH_DTYPES[cfg.dtype]
    parents, ranks = tree_parents_ranked(cfg.branching, N)
    max_rank = int(ranks.max()) + 1 if N else 1
    pos_parent = np.where(parents < 0, 0, parents + 1)
    if _is_cpu(device):
        gt = seed_stream(cfg.config_id, cfg.variant, STREAM_TARGET)
        target = torch.empty((B, N + 1, V), dtype=dt)
        for b in range(B):
            target[b] = torch.from_numpy(gt.standard_normal((N + 1, V)) * cfg.target_sigma).to(dt)
        stored = target.to(torch.float32).numpy()
        # stable descending order: equal logits keep the lower token id first
        top = np.argsort(-stored, axis=-1, kind="stable")[..., :max_rank]
        tokens = top[:, pos_parent, ranks].astype(np.int32)  # [B, N]
        gr = seed_stream(cfg.config_id, cfg.variant, STREAM_TREE_REPLACE)
        replace = gr.random((B, N)) < cfg.replace_prob
        rand_ids = gr.integers(0, V, size=(B, N), dtype=np.int64).astype(np.int32)
        tokens = np.where(replace, rand_ids, tokens)
        node_tokens = torch.from_numpy(tokens)
    else:
        gt = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_TARGET)
        target = torch.empty((B, N + 1, V), dtype=dt, device=device)
        per = max(1, (1 << 27) // max(1, (N + 1) * V))
        for b0 in range(0, B, per):
            b1 = min(B, b0 + per)
            target[b0:b1] = (torch.randn((b1 - b0, N + 1, V), generator=gt, device=device)
                             * cfg.target_sigma).to(dt)
        top = torch.empty((B, N + 1, max_rank), dtype=torch.int64, device=device)
        for b in range(B):
            order = torch.sort(target[b].to(torch.float32), dim=-1, descending=True, stable=True).indices
            top[b] = order[:, :max_rank]
        pp = torch.from_numpy(pos_parent.astype(np.int64)).to(device)
        rr = torch.from_numpy(ranks.astype(np.int64)).to(device)
        tokens = top[:, pp, rr].to(torch.int32)
        gr = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_TREE_REPLACE)
        replace = torch.rand((B, N), generator=gr, device=device) < cfg.replace_prob
        rand_ids = torch.randint(0, V, (B, N), generator=gr, device=device, dtype=torch.int64).to(torch.int32)
        node_tokens = torch.where(replace, rand_ids, tokens)
    return {
        "target": target,
        "node_tokens": node_tokens,
        "parents": torch.from_numpy(parents).to(device),
    }


def sample_tree_inputs(cfg: SampleTreeConfig, device="cpu", parents=None) -> dict:
    """Inputs of one sampling tree-verification call on ``device``.

    Keys: ``target``, ``draft [B,N+1,V]`` (position 0 = the root, position
    i+1 = node i; draft = target + N(0, draft_sigma^2), each rounded to the
    storage dtype on its own), ``node_tokens [B,N]`` int32 (node i drawn from
    the stored draft distribution at its parent's position at temperature T,
    Gumbel-max, siblings independently), ``parents [N]``, ``temperature [B]``,
    ``uniforms [B,N+1]`` in [0, 1) (column i tests node i, column N drives the
    final draw). Streams: 0 target, 1 draft noise, 2 token Gumbel noise,
    3 uniforms. ``parents`` (int array of length N) replaces the tree cut
    from ``cfg.branching``.
    """
    B, N, V = cfg.B, cfg.N, cfg.V
    dt = _TORCH_DTYPES[cfg.dtype]
    if parents is None:
        parents, _ = tree_parents_ranked(cfg.branching, N)
    else:
        parents = np.asarray(parents, dtype=np.int32)
        if parents.shape != (N,):
            raise ValueError(f"parents must have length N = {N}")
    pos_parent = torch.from_numpy(np.where(parents < 0, 0, parents + 1).astype(np.int64))
    T = torch.full((B,), float(cfg.temperature), dtype=torch.float32)
    if _is_cpu(device):
        gt = seed_stream(cfg.config_id, cfg.variant, STREAM_TARGET)
        gd = seed_stream(cfg.config_id, cfg.variant, STREAM_DRAFT_NOISE)
        target = torch.empty((B, N + 1, V), dtype=dt)
        draft = torch.empty((B, N + 1, V), dtype=dt)
        for b in range(B):
            t64 = gt.standard_normal((N + 1, V)) * cfg.target_sigma
            target[b] = torch.from_numpy(t64).to(dt)
            draft[b] = torch.from_numpy(t64 + gd.standard_normal((N + 1, V)) * cfg.draft_sigma).to(dt)
        gx = seed_stream(cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
        gu = seed_stream(cfg.config_id, cfg.variant, STREAM_UNIFORMS)
        uniforms = torch.from_numpy(gu.random((B, N + 1), dtype=np.float32))
    else:
        gt = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_TARGET)
        gd = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_NOISE)
        target = torch.empty((B, N + 1, V), dtype=dt, device=device)
        draft = torch.empty((B, N + 1, V), dtype=dt, device=device)
        per = max(1, (1 << 26) // max(1, (N + 1) * V))
        for b0 in range(0, B, per):
            b1 = min(B, b0 + per)
            t32 = torch.randn((b1 - b0, N + 1, V), generator=gt, device=device) * cfg.target_sigma
            target[b0:b1] = t32.to(dt)
            draft[b0:b1] = (t32 + torch.randn(t32.shape, generator=gd, device=device) * cfg.draft_sigma).to(dt)
            del t32
        gx = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
        gu = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_UNIFORMS)
        uniforms = torch.rand((B, N + 1), generator=gu, device=device, dtype=torch.float32)
        T = T.to(device)
        pos_parent = pos_parent.to(device)
    tokens = torch.empty((B, N), dtype=torch.int32, device=target.device)
    per_seq = max(1, (1 << 24) // max(1, N * V))
    for b0 in range(0, B, per_seq):
        b1 = min(B, b0 + per_seq)
        rows = draft[b0:b1][:, pos_parent]  # [nb, N, V]: each node's parent-position draft row
        tokens[b0:b1] = sample_draft_tokens_gumbel(rows, T[b0:b1], gx)
    return {"target": target, "draft": draft, "node_tokens": tokens,
            "parents": torch.from_numpy(parents).to(target.device), "temperature": T, "uniforms": uniforms}


# ----------------------------------------------------------------------------- LM-head chain inputs

def lm_head_chain_inputs(cfg: LMHeadConfig, device="cuda") -> dict:
    """All inputs of one LM-head chain-verification call on ``device`` (a GPU;
    the weights of the c2h workload are 2.1 GB).

    Keys: ``hidden [B,K+1,H]``, ``weight [V,H]``, ``draft [B,K,V]`` (bf16),
    ``draft_tokens [B,K]`` int32 (drawn from the stored draft logits at the
    temperature), ``temperature [B]`` and ``uniforms [B,K+1]`` float32.
    """
    B, K, V, H = cfg.B, cfg.K, cfg.V, cfg.H
    gh = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_HIDDEN)
    gw = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_WEIGHT)
    gd = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_WEIGHT)
    prior = torch.from_numpy(zipf_log_prior(V, cfg.zipf_s)).to(device=device, dtype=torch.float32)
    if cfg.exact:
        hidden = torch.randint(-3, 4, (B, K + 1, H), generator=gh, device=device).float()
        weight = torch.randint(-3, 4, (V, H), generator=gw, device=device).float()
        weight[:, H - 1] = torch.round(8.0 * prior)
        spread = math.sqrt((H - 1) * 4.0 * 4.0)  # sd of a sum of H-1 products of two uniform ints in [-3, 3]
        temperature = cfg.temperature * spread / cfg.target_sigma
    else:
        hidden = torch.randn((B, K + 1, H), generator=gh, device=device)
        weight = torch.randn((V, H), generator=gw, device=device) * (cfg.target_sigma / math.sqrt(H - 1))
        weight[:, H - 1] = prior
        temperature = cfg.temperature
    hidden[..., H - 1] = 1.0
    hidden = hidden.to(torch.bfloat16)
    weight = weight.to(torch.bfloat16)
    # the draft's head: perturbed weights on the same hidden states
    draft = torch.empty((B, K, V), dtype=torch.bfloat16, device=device)
    h_draft = hidden[:, :K].reshape(B * K, H).float()
    per = max(1, (1 << 28) // (4 * max(1, B * K)))  # vocabulary rows per chunk
    for v0 in range(0, V, per):
        v1 = min(V, v0 + per)
        w = weight[v0:v1].float()
        if cfg.exact:
            r = torch.rand(w.shape, generator=gd, device=device)
            w = w + (r < 0.2).float() - (r > 0.8).float()
        else:
            w = w + torch.randn(w.shape, generator=gd, device=device) * (cfg.draft_sigma / math.sqrt(H - 1))
        draft[:, :, v0:v1] = (h_draft @ w.T).reshape(B, K, v1 - v0).to(torch.bfloat16)
        del w
    temp = torch.full((B,), float(temperature), dtype=torch.float32, device=device)
    gx = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_DRAFT_TOKENS)
    tokens = sample_draft_tokens_gumbel(draft, temp, gx)
    gu = _torch_generator(device, cfg.config_id, cfg.variant, STREAM_UNIFORMS)
    uniforms = torch.rand((B, K + 1), generator=gu, device=device, dtype=torch.float32)
    return {"hidden": hidden, "weight": weight, "draft": draft, "draft_tokens": tokens, "temperature": temp,
            "uniforms": uniforms}
