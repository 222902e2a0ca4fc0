"""CPU oracle for speculative-sampling verification (float64 numpy).

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library. Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may import
or run it; the product path (the C-ABI library and its Python binding) never
does, and shares no code, table or helper with it.

It is the plain definition of what a verification step computes, evaluated in
float64 on the CPU with library primitives (``exp``, ``cumsum``, ``argmax``)
and no blocking, fusion or reordering. Sources, cited by page title and section:

* [Topologies] "Speculative Decoding & Draft Model Topologies: Slashing
  Enterprise LLM Latency by 3.5x in 2026", section 2 (speculative verification
  and rejection sampling: the acceptance-probability and residual equations,
  and the four-step timeline figure) and section 4 (EAGLE-2 tree figure).
* [Draft-and-Verify] "Speculative Decoding for LLM Inference: How
  Draft-and-Verify Accelerates Token Generation", sections "The draft-and-verify
  loop", "The correctness guarantee" and "How much speedup to expect".
* [At Scale] "Speculative Decoding at Scale: Latency Reduction in Distributed
  LLM Serving", the sequence diagram and section 1 (mathematical mechanics).
* [In Production] "Speculative Decoding in Production: How Small Draft Models &
  Medusa Heads Deliver 2x-3x LLM Speedups Without Accuracy Loss", section 2
  (rejection-sampling rules) and section 4 (tree verification, 2D masks).

Readings taken where the pages are silent or disagree (each is listed, with
its reason, in the design notes of the repository):

1. accept iff ``u < alpha`` with ``u`` in [0, 1) (one page writes ``<=``); a
   token with p(x) = 0 is never accepted, so alpha = 0 there; alpha = 1 when
   q(x) = 0 < p(x);
2. the same temperature scales target and draft logits of a sequence;
3. ``uniforms[b, K]`` drives the replacement / bonus draw;
4. inverse CDF over ascending token id: the first t with
   cumsum(w)[t] > u * sum(w); if rounding leaves none, the last t with w > 0;
5. a rejected position whose residual sums to 0 samples from p at that position;
6. greedy tree: argmax ties go to the lowest token id, deepest-node ties to the
   lowest node id; node i is verified at position i + 1, the root at 0;
7. the tree mask covers nodes only: M[i, j] = 1 iff j is i or an ancestor of i;
8. rows with an out-of-range token, a non-positive / non-finite temperature or
   a bad parent are reported with accept_len = -1 (library contract);
9. sampling tree verification: the children of a node are tried in ascending
   index against the current P, each rejection replacing P by its normalised
   residual against the node's draft distribution q; the walk stops at a node
   whose children are all rejected (or a leaf) and draws from P there.
"""
from __future__ import annotations

import numpy as np

FLAG_WINDOW = 1e-6  # a decision whose uniform lies this close to its threshold is flagged


# ----------------------------------------------------------------------------- distributions

def temperature_softmax(logits, temperature):
    """Distribution over the vocabulary (last axis): p(v) = exp(l_v / T) / sum_w exp(l_w / T).

    [Draft-and-Verify] "Why autoregressive decoding is slow" and "The
    draft-and-verify loop": each verified position yields a probability
    distribution over the vocabulary; [In Production] section 2: the guarantee
    holds at every temperature, so the logits are divided by T before the
    normalisation. ``temperature`` broadcasts against ``logits[..., 0]``.
    The maximum is subtracted before exponentiation (a rounding safeguard that
    leaves the ratio unchanged).
    """
    a = np.asarray(logits, dtype=np.float64) / np.asarray(temperature, dtype=np.float64)[..., None]
    a = a - a.max(axis=-1, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=-1, keepdims=True)


def entropy(p):
    """Shannon entropy in nats over the last axis: H = -sum_v p(v) ln p(v), 0 ln 0 = 0.

    [At Scale] section 3 (engineering recommendations): the speculation
    length K is to be tuned from the entropy of the predictions (lower K where
    the models diverge). The pages name the quantity without a formula; this
    is the textbook definition, applied to the temperature softmax p of one
    position.
    """
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return -terms.sum(axis=-1)


def acceptance_probability(p_x, q_x):
    """alpha = min(1, p(x) / q(x)) for a drafted token x.

    [Topologies] section 2, acceptance-probability equation; [Draft-and-Verify]
    "The correctness guarantee"; [In Production] section 2 (p >= q: always
    kept; p < q: kept with probability p/q). Edge readings: alpha = 0 when
    p(x) = 0, and alpha = 1 when q(x) = 0 < p(x).
    """
    p_x = np.asarray(p_x, dtype=np.float64)
    q_x = np.asarray(q_x, dtype=np.float64)
    safe_q = np.where(q_x > 0, q_x, 1.0)
    ratio = np.where(q_x > 0, p_x / safe_q, np.inf)
    return np.where(p_x > 0, np.minimum(1.0, ratio), 0.0)


def residual_weights(p, q):
    """Unnormalised residual max(0, p(v) - q(v)) at a rejected position.

    [Topologies] section 2, residual equation; [Draft-and-Verify] "The
    correctness guarantee" (normalised positive difference); [At Scale]
    section 1 (the relu form); [In Production] section 2.
    """
    return np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))


def inverse_cdf(weights, u):
    """Draw from the (unnormalised) ``weights`` over the last axis with uniform ``u``.

    Returns the first index t (ascending token id) with
    cumsum(weights)[t] > u * sum(weights), and if rounding leaves no such index,
    the last index with a positive weight. Also returns the two CDF boundaries
    around t in u-space (normalised), for flagging near-boundary draws.
    """
    w = np.asarray(weights, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    c = np.cumsum(w, axis=-1)
    total = c[..., -1]
    hit = c > (u * total)[..., None]
    t = np.argmax(hit, axis=-1)
    none = ~hit.any(axis=-1)
    if np.any(none):
        last_pos = w.shape[-1] - 1 - np.argmax((w > 0)[..., ::-1], axis=-1)
        t = np.where(none, last_pos, t)
    ti = t[..., None]
    hi = np.take_along_axis(c, ti, axis=-1)[..., 0]
    lo = np.where(t > 0, np.take_along_axis(c, np.maximum(ti - 1, 0), axis=-1)[..., 0], 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lo_u = np.where(total > 0, lo / total, 0.0)
        hi_u = np.where(total > 0, hi / total, 1.0)
    return t, lo_u, hi_u


# ----------------------------------------------------------------------------- draft-side sampling

def sample_rows(logits, temperature, uniforms):
    """Draw one token per row from its temperature softmax (the drafter's step).

    [In Production] section 2 (each step the draft model samples a candidate
    x ~ q(x)); [Draft-and-Verify] "The draft-and-verify loop" (the draft model
    proposes its tokens one position at a time). Readings 2 and 4: the row's
    temperature divides its logits, and the draw is the inverse CDF over
    ascending token id with the row's uniform, as for the replacement draw.

    Shapes: ``logits [R, V]``, ``temperature [R]`` (or None for T = 1),
    ``uniforms [R]``. Returns ``tokens [R]`` int64, ``prob [R]`` (q of the drawn
    token), and the drawn token's CDF boundaries ``lo_u, hi_u [R]`` in u-space
    (a uniform within FLAG_WINDOW of either boundary is a near-boundary draw).
    """
    logits = np.asarray(logits, dtype=np.float64)
    R = logits.shape[0]
    T = np.ones(R) if temperature is None else np.asarray(temperature, dtype=np.float64)
    q = temperature_softmax(logits, T)
    t, lo_u, hi_u = inverse_cdf(q, np.asarray(uniforms, dtype=np.float64))
    prob = np.take_along_axis(q, t[:, None], axis=1)[:, 0]
    return t.astype(np.int64), prob, lo_u, hi_u


# ----------------------------------------------------------------------------- chain verification

def verify_chain(target_logits, draft_logits, draft_tokens, temperature, uniforms, with_entropy=False):
    """One verification step of chain speculative sampling for a batch of sequences.

    Shapes: target ``[B, K+1, V]``, draft ``[B, K, V]``, draft_tokens ``[B, K]``,
    temperature ``[B]``, uniforms ``[B, K+1]``. For each sequence:

    1. p_k = softmax(target_k / T) for k = 0..K, q_k = softmax(draft_k / T)
       for k < K ([Topologies] section 2 timeline figure, step 2;
       [Draft-and-Verify] "The draft-and-verify loop").
    2. alpha_k = min(1, p_k(x_k) / q_k(x_k)); drafted token k is accepted iff
       u_k < alpha_k ([Topologies] section 2; [In Production] section 2).
    3. The candidates are checked in order and the first rejection ends the
       run: j = the first rejected k, or K if none ([Topologies] timeline
       step 3; [Draft-and-Verify] loop: the longest accepted prefix).
    4. If j < K, one token is drawn from the residual max(0, p_j - q_j) /
       sum(...) ([Topologies] residual equation; [At Scale] section 1); if
       j = K, a bonus token is drawn from p_K ([Draft-and-Verify] loop; [At
       Scale] diagram: the target adds one extra token). The draw uses u_K and the inverse
       CDF over ascending token id.
    5. Output: x_0..x_{j-1}, then the drawn token: between 1 and K+1 tokens
       ([Draft-and-Verify] loop).

    Step 1 is done here; steps 2 to 5 by :func:`verify_chain_distributions`,
    which also serves callers that verify the same distributions with several
    sets of uniforms.

    Returns a dict of numpy arrays: ``accept_len [B]`` (j, or -1 for an invalid
    row), ``out_tokens [B, K+1]`` (-1 after position j), ``p_draft``,
    ``q_draft [B, K]`` (p_k(x_k), q_k(x_k) for every k), ``residual_mass [B]``
    (sum max(0, p_j - q_j), -1 when all K are accepted), with ``with_entropy``
    ``entropy [B, 2K+1]`` (the entropy in nats of p_0 .. p_K, then of
    q_0 .. q_{K-1}), and the diagnostics listed under
    :func:`verify_chain_distributions`.
    """
    t = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_logits, dtype=np.float64)
    x = np.asarray(draft_tokens, dtype=np.int64)
    T = np.asarray(temperature, dtype=np.float64)
    B, K1, V = t.shape
    K = K1 - 1
    if d.shape != (B, K, V) or x.shape != (B, K) or T.shape != (B,):
        raise ValueError("inconsistent shapes")
    valid = chain_rows_valid(x, T, V)
    T_safe = np.where(valid, T, 1.0)

    # 1. target and draft distributions at every position
    p = temperature_softmax(t, T_safe[:, None])  # [B, K+1, V]
    q = temperature_softmax(d, T_safe[:, None])  # [B, K, V]
    res = verify_chain_distributions(p, q, x, uniforms, valid)
    if with_entropy:  # per-position entropy of every distribution of the step
        res["entropy"] = np.concatenate([entropy(p), entropy(q)], axis=1)
    return res


def chain_rows_valid(draft_tokens, temperature, V):
    """Rows the library verifies (reading 8): a positive finite temperature and
    every drafted token in [0, V)."""
    x = np.asarray(draft_tokens, dtype=np.int64)
    T = np.asarray(temperature, dtype=np.float64)
    valid = np.isfinite(T) & (T > 0)
    if x.shape[1]:
        valid &= np.all((x >= 0) & (x < V), axis=1)
    return valid


def verify_chain_distributions(p, q, draft_tokens, uniforms, valid):
    """Steps 2 to 5 of :func:`verify_chain` on given distributions.

    ``p [B, K+1, V]`` and ``q [B, K, V]`` are the target and draft
    distributions (step 1), ``draft_tokens [B, K]``, ``uniforms [B, K+1]``,
    ``valid [B]`` (see :func:`chain_rows_valid`). Returns the outputs of
    :func:`verify_chain` and these diagnostics: ``alpha [B, K]``,
    ``margin_accept [B, K]`` (|u_k - alpha_k| for the checked positions, +inf
    for the others), ``margin_sample [B]`` (distance of u_K to the nearest CDF
    boundary of the drawn token), ``flagged [B]`` (a margin below
    FLAG_WINDOW), ``valid [B]``, and ``flag_rate [B]``: for uniforms drawn
    afresh, about how likely a row with this j is to be flagged: for each
    checked accept test the length of [alpha_k - FLAG_WINDOW, alpha_k +
    FLAG_WINDOW] inside [0, 1), plus, for the draw, sum_v min(w_v / sum(w),
    2 FLAG_WINDOW) over the normalised sampling weights (the chance that u_K
    lands within the window of a boundary of the token it selects).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    x = np.asarray(draft_tokens, dtype=np.int64)
    u = np.asarray(uniforms, dtype=np.float64)
    valid = np.asarray(valid, dtype=bool)
    B, K1, V = p.shape
    K = K1 - 1
    if q.shape != (B, K, V) or x.shape != (B, K) or u.shape != (B, K1) or valid.shape != (B,):
        raise ValueError("inconsistent shapes")
    x_safe = np.where((x >= 0) & (x < V), x, 0)

    # 2. acceptance probability of each drafted token
    bi = np.arange(B)[:, None]
    ki = np.arange(K)[None, :]
    p_x = p[bi, ki, x_safe]
    q_x = q[bi, ki, x_safe]
    alpha = acceptance_probability(p_x, q_x)
    accepted = u[:, :K] < alpha

    # 3. first rejection
    rejected = ~accepted
    j = np.where(rejected.any(axis=1), np.argmax(rejected, axis=1), K) if K else np.zeros(B, np.int64)

    # 4. sampling weights: residual at j < K, p_K for the bonus
    rows = np.arange(B)
    p_j = p[rows, j]  # [B, V]; j == K selects the bonus position
    q_j = q[rows, np.minimum(j, K - 1)] if K else np.zeros_like(p_j)
    is_residual = j < K
    r = residual_weights(p_j, q_j)
    s = r.sum(axis=1)
    weights = np.where((is_residual & (s > 0))[:, None], r, p_j)
    residual_mass = np.where(is_residual, s, -1.0)
    token, lo_u, hi_u = inverse_cdf(weights, u[:, K])

    # 5. emitted tokens: the accepted prefix, then the drawn token
    pos = np.arange(K1)[None, :]
    x_pad = np.concatenate([x, np.zeros((B, 1), dtype=np.int64)], axis=1)
    out = np.where(pos < j[:, None], x_pad, -1)
    out[rows, j] = token

    # diagnostics for the parity comparison
    checked = ki <= j[:, None]  # positions whose accept test decided the outcome
    margin_accept = np.where(checked, np.abs(u[:, :K] - alpha), np.inf)
    margin_sample = np.minimum(u[:, K] - lo_u, hi_u - u[:, K])
    flagged = (margin_accept.min(axis=1, initial=np.inf) < FLAG_WINDOW) | (margin_sample < FLAG_WINDOW)
    with np.errstate(divide="ignore", invalid="ignore"):
        wsum = weights.sum(axis=1, keepdims=True)
        wn = np.where(wsum > 0, weights / np.where(wsum > 0, wsum, 1.0), 0.0)
    window = np.minimum(alpha + FLAG_WINDOW, 1.0) - np.maximum(alpha - FLAG_WINDOW, 0.0)  # inside [0, 1)
    flag_rate = np.minimum(wn, 2 * FLAG_WINDOW).sum(axis=1) + np.where(checked, window, 0.0).sum(axis=1)

    accept_len = np.where(valid, j, -1).astype(np.int64)
    out[~valid] = -1
    residual_mass[~valid] = -1.0
    return {
        "accept_len": accept_len,
        "out_tokens": out,
        "p_draft": p_x,
        "q_draft": q_x,
        "residual_mass": residual_mass,
        "alpha": alpha,
        "margin_accept": margin_accept,
        "margin_sample": margin_sample,
        "flagged": flagged & valid,
        "flag_rate": np.where(valid, flag_rate, 0.0),
        "valid": valid,
    }


# ----------------------------------------------------------------------------- the target's LM head

def round_to_bf16(x):
    """Round to the nearest bfloat16 value, ties to even, returned as float64.

    bfloat16 keeps 8 significant bits (the upper half of a binary32). A
    finite x = m 2^e with m in [1/2, 1) becomes rint(m 2^8) 2^(e-8), rint
    rounding half to even. Values beyond the binary32 exponent range are
    outside this oracle's use (the synthetic logits are small).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def lm_head_logits(hidden, weight):
    """The target's logits at every verified position: logits[m, v] =
    sum_h hidden[m, h] weight[v, h], in float64.

    [Topologies] section 2 timeline figure, step 2 (the target model scores
    every drafted position in one forward pass); [Draft-and-Verify] "Why
    autoregressive decoding is slow" and "The draft-and-verify loop" (each
    verified position yields a distribution over the vocabulary). The pages
    do not print the model; the last layer is taken as a plain linear map
    from the final hidden state to one logit per vocabulary entry.
    ``hidden [..., H]`` (any leading shape), ``weight [V, H]``.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return h @ w.T


def verify_chain_lm_head(hidden, weight, draft_logits, draft_tokens, temperature, uniforms, with_entropy=False):
    """Chain verification with the target's logits made by its LM head:
    the logits of ``hidden [B, K+1, H]`` through ``weight [V, H]``
    (:func:`lm_head_logits`), stored as bfloat16 (:func:`round_to_bf16`,
    the precision the target hands to verification), then
    :func:`verify_chain` on them with the draft's logits. Returns
    verify_chain's dict plus ``target_logits [B, K+1, V]`` (the stored
    values, float64)."""
    t = round_to_bf16(lm_head_logits(hidden, weight))
    res = verify_chain(t, draft_logits, draft_tokens, temperature, uniforms, with_entropy=with_entropy)
    res["target_logits"] = t
    return res


# ----------------------------------------------------------------------------- tree verification

def _check_parents(parents):
    parents = np.asarray(parents, dtype=np.int64)
    for i, par in enumerate(parents):
        if not (par == -1 or 0 <= par < i):
            return False
    return True


def node_depths(parents):
    """Depth of every node: 1 for a child of the root, parent's depth + 1 otherwise."""
    parents = np.asarray(parents, dtype=np.int64)
    depth = np.zeros(len(parents), dtype=np.int64)
    for i, par in enumerate(parents):
        depth[i] = 1 if par < 0 else depth[par] + 1
    return depth


def verify_tree_greedy(target_logits, node_tokens, parents):
    """Greedy (argmax-matching) verification of a candidate tree, per sequence.

    target ``[B, N+1, V]``: position 0 holds the target's logits after the root
    (the last accepted token), position i+1 those after node i. node_tokens
    ``[B, N]``, parents ``[N]`` (-1 = child of the root, else an earlier node).

    [Topologies] section 4 figure: every node of the candidate tree is checked
    in one target pass and the longest accepted path along the tree is kept;
    [In Production] section 4: a tree of competing branches verified at once;
    [At Scale] sequence diagram: tokens that match the target are accepted and
    the target supplies one more token. A node is accepted when its token equals
    the target's argmax at its parent's position and its parent is accepted (or
    is the root). The deepest accepted node ends the path (lowest index on
    ties); the next token is the argmax at that node's position.

    Returns ``accept_len [B]`` (depth of the deepest accepted node, -1 for an
    invalid row), ``path_nodes [B, N]`` (node ids, root side first, -1 padded),
    ``next_token [B]`` and ``argmax [B, N+1]``.
    """
    t = np.asarray(target_logits)
    tok = np.asarray(node_tokens, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    B, N1, V = t.shape
    N = N1 - 1
    if tok.shape != (B, N) or parents.shape != (N,):
        raise ValueError("inconsistent shapes")
    accept_len = np.full(B, -1, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    nxt = np.full(B, -1, dtype=np.int64)
    g = np.argmax(t, axis=-1)  # first occurrence on ties: lowest token id
    if not _check_parents(parents):
        return {"accept_len": accept_len, "path_nodes": path, "next_token": nxt, "argmax": g}
    depth = node_depths(parents)
    for b in range(B):
        if N and not np.all((tok[b] >= 0) & (tok[b] < V)):
            continue
        acc = np.zeros(N, dtype=bool)
        for i in range(N):
            par = parents[i]
            pos = 0 if par < 0 else par + 1
            acc[i] = (tok[b, i] == g[b, pos]) and (par < 0 or acc[par])
        best = -1
        for i in range(N):
            if acc[i] and (best < 0 or depth[i] > depth[best]):
                best = i
        if best < 0:
            accept_len[b] = 0
            nxt[b] = g[b, 0]
            continue
        chain = []
        k = best
        while k >= 0:
            chain.append(k)
            k = parents[k]
        chain.reverse()
        accept_len[b] = len(chain)
        path[b, :len(chain)] = chain
        nxt[b] = g[b, best + 1]
    return {"accept_len": accept_len, "path_nodes": path, "next_token": nxt, "argmax": g}


def children_in_order(parents):
    """Children of the root (key -1) and of every node, in ascending node index."""
    parents = np.asarray(parents, dtype=np.int64)
    kids = {-1: []}
    for i in range(len(parents)):
        kids[i] = []
    for i, par in enumerate(parents):
        kids[int(par)].append(i)
    return kids


def verify_tree_stochastic(target_logits, draft_logits, node_tokens, parents, temperature, uniforms):
    """Lossless sampling verification of a candidate tree, per sequence.

    The pages verify a tree of competing branches in one target pass and keep
    the longest accepted path ([Topologies] section 4 figure; [In Production]
    section 4, after SpecInfer), and state the per-token rule for sampling
    (acceptance probability min(1, p/q), residual max(0, p - q) normalised;
    [Topologies] section 2; [In Production] section 2). They give no rule for
    several candidates at one position. Reading taken (multi-step speculative
    sampling, the rule of the SpecInfer paper the pages cite): at the current
    node, with P = p (the target's distribution at its position) and q (the
    draft's distribution its children were drawn from, i.i.d.), the children
    are tried in ascending node index; child v with token x is accepted iff
    u_v < min(1, P(x) / q(x)); a rejection replaces P by
    max(0, P - q) / sum(max(0, P - q)) (unchanged if that sum is 0) before the
    next child; an accepted child becomes the current node; when no child is
    accepted (or the node is a leaf), one token is drawn from P by the inverse
    CDF with the final uniform. With one child per node this is chain
    verification exactly.

    Shapes: target and draft ``[B, N+1, V]`` (position 0: after the root,
    position i+1: after node i; the draft row at a node's position is the
    distribution its children were sampled from), node_tokens ``[B, N]``,
    parents ``[N]``, temperature ``[B]`` (the same T for p and q), uniforms
    ``[B, N+1]`` (column v tests node v, column N drives the final draw).
    Returns ``accept_len [B]`` (-1 for an invalid row), ``path_nodes [B, N]``,
    ``next_token [B]``, ``emitted [B, N+1]`` (the path's tokens then the drawn
    token, -1 padded), ``flagged [B]`` (a tested uniform within FLAG_WINDOW of
    its acceptance probability, or the final uniform within FLAG_WINDOW of a
    CDF boundary of the drawn token), ``valid [B]``, ``tests [B]`` (how many
    children were tested), ``margin [B]`` (the smallest of those distances).
    """
    t = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_logits, dtype=np.float64)
    tok = np.asarray(node_tokens, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    T = np.asarray(temperature, dtype=np.float64)
    u = np.asarray(uniforms, dtype=np.float64)
    B, N1, V = t.shape
    N = N1 - 1
    if d.shape != t.shape or tok.shape != (B, N) or parents.shape != (N,) or T.shape != (B,) or u.shape != (B, N1):
        raise ValueError("inconsistent shapes")
    accept_len = np.full(B, -1, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    nxt = np.full(B, -1, dtype=np.int64)
    emitted = np.full((B, N1), -1, dtype=np.int64)
    flagged = np.zeros(B, dtype=bool)
    valid = np.zeros(B, dtype=bool)
    tests = np.zeros(B, dtype=np.int64)
    margin = np.full(B, np.inf)
    if not _check_parents(parents):
        return {"accept_len": accept_len, "path_nodes": path, "next_token": nxt, "emitted": emitted,
                "flagged": flagged, "valid": valid, "tests": tests, "margin": margin}
    kids = children_in_order(parents)
    for b in range(B):
        if not (np.isfinite(T[b]) and T[b] > 0) or (N and not np.all((tok[b] >= 0) & (tok[b] < V))):
            continue
        valid[b] = True
        node, pos, chain = -1, 0, []
        while True:
            P = temperature_softmax(t[b, pos], T[b])
            q = temperature_softmax(d[b, pos], T[b])
            taken = None
            for v in kids[node]:
                x = tok[b, v]
                alpha = float(acceptance_probability(P[x], q[x]))
                tests[b] += 1
                margin[b] = min(margin[b], abs(u[b, v] - alpha))
                if u[b, v] < alpha:
                    taken = v
                    break
                r = residual_weights(P, q)
                s = r.sum()
                if s > 0:
                    P = r / s
            if taken is None:
                break
            chain.append(taken)
            node, pos = taken, taken + 1
        drawn, lo, hi = inverse_cdf(P, u[b, N])
        accept_len[b] = len(chain)
        path[b, :len(chain)] = chain
        nxt[b] = int(drawn)
        emitted[b, :len(chain)] = tok[b, chain] if chain else []
        emitted[b, len(chain)] = int(drawn)
        flagged[b] = margin[b] < FLAG_WINDOW or min(u[b, N] - lo, hi - u[b, N]) < FLAG_WINDOW
    return {"accept_len": accept_len, "path_nodes": path, "next_token": nxt, "emitted": emitted,
            "flagged": flagged, "valid": valid, "tests": tests, "margin": margin}


def tree_mask(parents):
    """Tree attention mask over the candidate nodes: M[i, j] = 1 iff j == i or j is an ancestor of i.

    [Topologies] section 4 figure (all nodes verified together through a 2D
    tree-masked attention); [In Production] section 4 (a custom 2D causal mask
    lets one pass verify every branch). Returns uint8 ``[N, N]``; raises
    ValueError on a parent that is not -1 or an earlier node.
    """
    parents = np.asarray(parents, dtype=np.int64)
    if not _check_parents(parents):
        raise ValueError("parents[i] must be -1 or in [0, i)")
    N = len(parents)
    m = np.zeros((N, N), dtype=np.uint8)
    for i in range(N):
        k = i
        while k >= 0:
            m[i, k] = 1
            k = parents[k]
    return m
