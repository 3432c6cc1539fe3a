"""Float64 CPU oracle for the fixed-budget KV-cache evict-and-attend decode step.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module. The library and
its Python binding never do; the oracle shares no code with them (its inputs
come from the separate ``synthetic`` input module).

What it computes, step by step, in the pages' notation:

* Scorer. KVpop ("KVpop - Key-Value Cache Compression with Predictive Online
  Pruning"), section 3.3 "Stateless scorers" and Appendix E.1-E.2, Eq. (35)-(36):
  a per-KV-head two-layer MLP over the concatenation x = [k; v] of a cached
  token's key and value. Fast KVzip ("Fast KVzip: Efficient and Accurate LLM
  Inference with Gated KV Eviction"), section 3.1 "Formulation": a per-KV-head
  gate on the layer's hidden state with output in [0, 1] (here a linear map
  followed by a sigmoid). Scores are ranked in float32 (KVpop Appendix F,
  "Training details": top-k ranking and selection in float32).
* Prefill selection and masked prefill attention. KVpop section 3.2
  "Running top-k sparse attention" and Appendix C.1-C.2, Eq. (26): each
  query position q keeps the sinks, its recent window and the eligible
  tokens whose static-priority rank is within the rank tau_q of the k-th
  best eligible token; attention over the prompt uses that mask.
* Stateful scorer. KVpop section 3.3 "Stateful scorers", Appendix A and
  E.3-E.4, Eq. (10)-(11) and (37)-(42): per KV head, Hedgehog features of
  small projections of x = [k; v], a gated matrix memory C and normaliser z
  updated by every token, and a delayed read-out: after absorbing position q
  the token at q - W is scored from the state that has seen q.
* Sink-attention gate. Fast KVzip section 3.4 "Low-Rank Sink Attention":
  low-rank normalised projections of the hidden state give per-KV-head keys
  and per-query-head queries; each query weighs the token's key against a
  fixed set of sink keys and a learnable denominator term.
* Retention rule. KVpop section 3, Eq. (1) B = s + w + k; section 3.1 Eq. (4)
  eligible set E(q) = {t | s <= t <= q - w}; Appendix C.1 Eq. (26) retained
  set = sinks, recent window, and the top-k eligible tokens.
* Periodic eviction. ForesightKV summary page ("ForesightKV: Optimizing KV
  Cache Eviction for Reasoning Models by Learning Long-Term Contribution"),
  "Methodology in plain English": the cache is checked every L new tokens;
  when it reaches B + L, the recent tokens are protected and the lowest-scored
  pairs are evicted back to the budget. Fast KVzip Appendix A.5: buffered
  scoring of the pending tokens and eviction of as many entries.
* Attention over the retained entries. KVpop Appendix C (decoding attends over
  the compact cache) and Appendix D.1, Eq. (27)-(29): logits <q, k>/sqrt(d_k),
  log-sum-exp normaliser, probabilities exp(logit - LSE).

Readings where the pages leave a step open (also listed in the design notes):

* The window holds the W most recent tokens including the newest one
  (KVpop Appendix C.1, set 2: q - t < w), so eligible tokens satisfy
  S <= t <= P - W for newest position P. Sinks, window and candidates are
  identified by position, not by slot.
* Compaction keeps kept entries below the new count in place and moves the
  kept entries above it into the freed slots, both in ascending slot order.
* Eviction fires after prefill when n0 > B, and during decode when the cache
  count n reaches B + L; it evicts n - B entries, so the cache holds B after
  every eviction and B..B+L-1 between evictions.
* Ties: among equal float32 scores the older (lower position) token is
  evicted first; -0.0 is treated as +0.0. Non-finite scores are outside the
  contract (asserted here).
* Temporal decay (optional, per KV head): decay step n = 1 only (KVpop Table
  3 uses n = 1), ranking by the static priority of Eq. (20) in float32.
* Query head j reads KV head floor(j / G) (contiguous GQA groups).
* Sink-attention gate (the page's equation is not legible; these follow its
  prose): RMS normalisation with eps 1e-6 after each projection, logits
  scaled by 1/sqrt(D'), the token's own term in the denominator (so the
  gate lies in [0, 1] for b >= 0 and the no-denominator variant is a
  sigmoid), one shared set of sink keys per layer, and the maximum over the
  G query heads of a KV head.
* Stochastic eviction (ForesightKV): the pool is the 2r lowest-ranked
  candidates for r evictions; the page weights the draws by the negated
  scores, read here as a softmax over -key (a multinomial over logits, the
  form its policy-gradient training needs, defined for any real score); the
  r draws without replacement are realised by Gumbel-top-k with the noise
  passed in, sums rounded to float32, equal sums evicting the older token.
* Stateful scorer: the Hedgehog variant with projection width P = d/2
  (features of 2P entries), scalar affine gate preactivations with biases, no
  output gate, soft-cap, norm or skip connection; the read-out delay equals
  the window W; the plain (unstabilised) recurrence in float64.

Parity pins: every function here is pinned by tests in
``tests/test_oracle_pins.py`` to facts other than its own formula
(hand-computed fixtures, library routines, brute force, closed forms and
invariants). No function is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Policy", "mlp_score", "gate_score", "score_to_f32", "static_priority",
    "hedgehog", "MlstmWeights", "mlstm_features", "mlstm_readout",
    "MlstmScorer", "mlstm_scores_parallel",
    "prefill_ranks", "prefill_cutoffs", "prefill_mask", "prefill_attention",
    "rms_norm", "SinkGateWeights", "sink_gate_score", "select_keep_stochastic",
    "eligible_mask",
    "select_keep", "compaction_sources", "compact_slice", "attention_probs", "decode_attention", "OracleLayer",
    "closed_form_retained", "cache_bytes_per_token",
]


@dataclass(frozen=True)
class Policy:
    """Budget B, sinks S, window W and eviction length L (KVpop Eq. (1);
    ForesightKV summary, periodic eviction with length L). ``log_gamma``
    optionally holds one log decay factor per KV head (KVpop Eq. (5) with
    decay step n = 1; ranking by the static priority of Eq. (20))."""

    budget: int
    sinks: int
    window: int
    evict_len: int
    log_gamma: Optional[tuple] = None

    @property
    def k(self) -> int:
        """Long-range top-k budget k = B - s - w (KVpop Eq. (1))."""
        return self.budget - self.sinks - self.window

    def check(self) -> None:
        if self.sinks < 0 or self.window < 0 or self.evict_len < 1:
            raise ValueError("policy: S, W must be >= 0 and L >= 1")
        if self.k < 0:
            raise ValueError("policy: B must be >= S + W")


# ---------------------------------------------------------------------------
# Scorers
# ---------------------------------------------------------------------------

def _act(a: np.ndarray, act: str) -> np.ndarray:
    if act == "relu":
        return np.maximum(a, 0.0)
    if act == "silu":
        # SiLU(a) = a * sigmoid(a) (KVpop section 3.3 uses SiLU).
        return a / (1.0 + np.exp(-a))
    raise ValueError(act)


def mlp_score(k: np.ndarray, v: np.ndarray, w1: np.ndarray, b1: np.ndarray,
              w2: np.ndarray, b2: float, act: str = "relu") -> np.ndarray:
    """Stateless head-wise MLP score of each token (KVpop section 3.3 and
    Appendix E.2, Eq. (36)), input x = [k; v] (Appendix E.1, Eq. (35)).

    k, v: [..., d]; w1: [hidden, 2d] (row j = input weights of hidden unit
    j); b1: [hidden]; w2: [hidden]; b2: scalar. Returns float64 [...].
    """
    x = np.concatenate([np.asarray(k, np.float64), np.asarray(v, np.float64)],
                       axis=-1)
    a = x @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64)
    h = _act(a, act)
    return h @ np.asarray(w2, np.float64) + float(b2)


def gate_score(hidden: np.ndarray, w: np.ndarray, b: float = 0.0
               ) -> np.ndarray:
    """Per-KV-head gate on a token's hidden state (Fast KVzip section 3.1,
    g_l : R^D -> [0, 1]^H): sigmoid(w . x + b). hidden [..., D], w [D]."""
    a = np.asarray(hidden, np.float64) @ np.asarray(w, np.float64) + float(b)
    return 1.0 / (1.0 + np.exp(-a))


def hedgehog(y: np.ndarray) -> np.ndarray:
    """Hedgehog feature map in softmax form (KVpop Appendix A): [softmax(y);
    softmax(-y)] over the last (feature) axis."""
    y = np.asarray(y, np.float64)

    def softmax(u):
        e = np.exp(u - u.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    return np.concatenate([softmax(y), softmax(-y)], axis=-1)


@dataclass
class MlstmWeights:
    """One KV head's stateful scorer (KVpop section 3.3 "Stateful scorers",
    Appendix A and E.3-E.4): projections W_q, W_k, W_v [P][2d] of
    x = [k; v], input/forget gate weights w_i, w_f [2d] and biases, readout
    a [P] and bias b."""

    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wi: np.ndarray
    wf: np.ndarray
    bi: float
    bf: float
    a: np.ndarray
    b: float


def mlstm_features(x: np.ndarray, w: MlstmWeights):
    """Per-token read/write features (KVpop Eq. (37), (40)): q~ = phi(W_q x),
    k~ = phi(W_k x), v~ = W_v x, input gate i = exp(w_i . x + b_i), forget
    gate f = sigmoid(w_f . x + b_f). x [..., 2d]."""
    x = np.asarray(x, np.float64)
    qf = hedgehog(x @ np.asarray(w.wq, np.float64).T)
    kf = hedgehog(x @ np.asarray(w.wk, np.float64).T)
    vf = x @ np.asarray(w.wv, np.float64).T
    ig = np.exp(x @ np.asarray(w.wi, np.float64) + w.bi)
    fg = 1.0 / (1.0 + np.exp(-(x @ np.asarray(w.wf, np.float64) + w.bf)))
    return qf, kf, vf, ig, fg


def mlstm_readout(qf_u: np.ndarray, C: np.ndarray, z: np.ndarray,
                  w: MlstmWeights) -> float:
    """Delayed readout h = (q~_u^T C_q) / (q~_u^T z_q) (KVpop Eq. (41)) and
    raw score a^T SiLU(h) + b (Eq. (42), without the optional norm)."""
    h = (qf_u @ C) / (qf_u @ z)
    return float(np.dot(np.asarray(w.a, np.float64), h / (1.0 + np.exp(-h))) + w.b)


class MlstmScorer:
    """The recurrent scorer state of one KV head: matrix memory C [2P][P]
    and normaliser z [2P] (KVpop Eq. (38)-(39)), updated token by token in
    plain (unstabilised) float64. At query position q the token u = q - W
    leaves the window and is scored from the state that has absorbed token
    q (Appendix E.4)."""

    def __init__(self, w: MlstmWeights, window: int):
        self.w, self.window = w, window
        P = np.asarray(w.wv).shape[0]
        self.C = np.zeros((2 * P, P))
        self.z = np.zeros(2 * P)
        self.qf = {}       # q~ of tokens still waiting for their readout
        self.q = -1

    def push(self, x: np.ndarray):
        """Absorb token q = previous + 1 with input x [2d]; return
        (u, score) for the token leaving the window, or None."""
        self.q += 1
        qf, kf, vf, ig, fg = mlstm_features(x, self.w)
        self.C = fg * self.C + ig * np.outer(kf, vf)
        self.z = fg * self.z + ig * kf
        self.qf[self.q] = qf
        u = self.q - self.window
        if u < 0:
            return None
        return u, mlstm_readout(self.qf.pop(u), self.C, self.z, self.w)


def mlstm_scores_parallel(x: np.ndarray, w: MlstmWeights, window: int
                          ) -> np.ndarray:
    """The same scores in parallel form (KVpop Appendix A: the recurrent and
    parallel views are equivalent): with D[q, t] = i_t prod_{t<j<=q} f_j
    for t <= q, token u read at q = u + W gets
    h = sum_t D[q, t] (q~_u . k~_t) v~_t / sum_t D[q, t] (q~_u . k~_t).
    x [n][2d]; returns float64 scores of tokens 0..n-1-W."""
    qf, kf, vf, ig, fg = mlstm_features(x, w)
    n = x.shape[0]
    logf = np.log(fg)
    cum = np.concatenate([[0.0], np.cumsum(logf)])   # cum[j] = sum_{<j}
    out = np.empty(max(n - window, 0))
    for u in range(n - window):
        q = u + window
        t = np.arange(q + 1)
        decay = ig[t] * np.exp(cum[q + 1] - cum[t + 1])
        sim = kf[t] @ qf[u]
        num = (decay * sim) @ vf[t]
        den = (decay * sim).sum()
        h = num / den
        out[u] = float(np.dot(np.asarray(w.a, np.float64),
                              h / (1.0 + np.exp(-h))) + w.b)
    return out


def rms_norm(y: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """Weighted normalisation over the last axis (the per-head RMS norm with
    a learnable per-feature weight that Fast KVzip section 3.4 applies after
    the gate projections): weight * y / sqrt(mean(y^2) + eps)."""
    y = np.asarray(y, np.float64)
    return np.asarray(weight, np.float64) * y / np.sqrt(
        np.mean(y * y, axis=-1, keepdims=True) + eps)


@dataclass
class SinkGateWeights:
    """One layer's low-rank sink-attention gate (Fast KVzip section 3.4,
    "Low-Rank Sink Attention"): projections W_k [H][D'][D] and
    W_q [H][G][D'][D] of the hidden state, the normalisation weights
    g_k, g_q [D'], the layer's S sink keys [S][D'] and the learnable
    denominator terms b [H][G]."""

    wk: np.ndarray
    wq: np.ndarray
    gk: np.ndarray
    gq: np.ndarray
    sinks: np.ndarray
    b: np.ndarray
    eps: float = 1e-6


def sink_gate_score(hidden: np.ndarray, w: SinkGateWeights) -> np.ndarray:
    """Per-KV-head gate scores of tokens with hidden states hidden [n][D]
    (Fast KVzip section 3.4): k_h = norm(W_k[h] x), q_j = norm(W_q[j] x);
    with logits a_j = q_j . k_h / sqrt(D') and c_jr = q_j . k_sink^r /
    sqrt(D'), query head j gives exp(a_j) / (exp(a_j) + sum_r exp(c_jr) +
    b_j) in [0, 1] (the variant without a learnable denominator sets
    sum_r exp(c_jr) + b_j = 1, i.e. sigmoid(a_j)); the KV head's score is the
    maximum over its G query heads. Returns [n][H]."""
    x = np.asarray(hidden, np.float64)
    wk = np.asarray(w.wk, np.float64)
    wq = np.asarray(w.wq, np.float64)
    H, G, dp = wq.shape[0], wq.shape[1], wq.shape[2]
    k = rms_norm(np.einsum("hpd,nd->nhp", wk, x), w.gk, w.eps)      # [n][H][D']
    q = rms_norm(np.einsum("hgpd,nd->nhgp", wq, x), w.gq, w.eps)    # [n][H][G][D']
    a = np.einsum("nhgp,nhp->nhg", q, k) / np.sqrt(dp)
    c = np.einsum("nhgp,rp->nhgr", q, np.asarray(w.sinks, np.float64)) / np.sqrt(dp)
    m = np.maximum(a, c.max(axis=-1) if c.shape[-1] else -np.inf)
    ea = np.exp(a - m)
    den = ea + np.exp(c - m[..., None]).sum(axis=-1) + \
        np.asarray(w.b, np.float64)[None] * np.exp(-m)
    return (ea / den).max(axis=-1)


def score_to_f32(s: np.ndarray) -> np.ndarray:
    """Scores are ranked in float32 (KVpop Appendix F). -0.0 becomes +0.0."""
    s32 = np.asarray(s, dtype=np.float64).astype(np.float32)
    if not np.all(np.isfinite(s32)):
        raise ValueError("non-finite score: outside the contract")
    s32 = s32 + np.float32(0.0)  # -0.0 + 0.0 == +0.0 in round-to-nearest
    return s32


# ---------------------------------------------------------------------------
# Selection and compaction
# ---------------------------------------------------------------------------

def static_priority(score32: np.ndarray, pos: np.ndarray,
                    log_gamma: Optional[float]) -> np.ndarray:
    """Ranking key with temporal decay, KVpop Appendix B.3: for decay step
    n = 1 the effective score r + (q - t) log(gamma) (Eq. (18)-(19)) ranks
    eligible tokens like the static priority r - t log(gamma) (Eq. (20)),
    since q log(gamma) is common to all of them. Ranking is in float32
    (Appendix F): the product t * log(gamma) is rounded to float32, then the
    difference. Without decay the key is the score itself."""
    s = np.asarray(score32, dtype=np.float32)
    if log_gamma is None:
        return s
    prod = np.asarray(pos).astype(np.float32) * np.float32(log_gamma)
    return (s - prod).astype(np.float32)


def eligible_mask(pos: np.ndarray, sinks: int, window: int) -> np.ndarray:
    """Entries that may be evicted: position t with S <= t <= P - W, where P
    is the newest position present (KVpop Eq. (4), the eligible set E(P));
    the others are the sink tokens and the recent window."""
    pos = np.asarray(pos)
    if pos.size == 0:
        return np.zeros(0, dtype=bool)
    newest = pos.max()
    return (pos >= sinks) & (pos <= newest - window)


def select_keep(score32: np.ndarray, pos: np.ndarray, length: int,
                n_keep: int, sinks: int, window: int,
                log_gamma: Optional[float] = None) -> np.ndarray:
    """Slots kept when a cache slice of ``length`` entries is cut to
    ``n_keep`` entries.

    Candidates are the entries of the eligible set E(P) (``eligible_mask``).
    The length - n_keep candidates with the smallest (float32 ranking key,
    position) are evicted; every other entry is kept (KVpop Eq. (26): sinks,
    recent window and the top-k eligible tokens). The key is the score, or
    the static priority under temporal decay (``static_priority``).

    Returns the kept slot indices in ascending order (int64).
    """
    pos = np.asarray(pos)[:length]
    score32 = static_priority(np.asarray(score32, dtype=np.float32)[:length],
                              pos, log_gamma)
    if n_keep >= length:
        return np.arange(length, dtype=np.int64)
    r = length - n_keep
    cand = np.nonzero(eligible_mask(pos, sinks, window))[0]
    if cand.size < r:
        raise ValueError("not enough eligible entries to evict")
    s = score32[cand] + np.float32(0.0)
    order = np.lexsort((pos[cand], s))      # ascending score, then position
    evicted = np.zeros(length, dtype=bool)
    evicted[cand[order[:r]]] = True
    return np.nonzero(~evicted)[0].astype(np.int64)


def select_keep_stochastic(score32: np.ndarray, pos: np.ndarray,
                           length: int, n_keep: int, sinks: int, window: int,
                           gumbel: np.ndarray,
                           log_gamma: Optional[float] = None) -> np.ndarray:
    """Slots kept under ForesightKV's stochastic eviction (summary page,
    "Key Contributions" item 4 and "Methodology in Plain English"): with
    r = length - n_keep entries to evict, the 2r lowest-ranked candidates
    (the order of ``select_keep``; all candidates if fewer) form the pool,
    and r of them are drawn without replacement with probability
    proportional to exp(-key), key being the ranking key of
    ``select_keep``.

    The draw is the Gumbel-top-k realisation of that sampling (successive
    draws without replacement from a softmax equal the r largest of
    logit + independent standard Gumbel noise): ``gumbel[slot]`` is the
    noise of the entry in that slot, passed in. Each pool entry gets the
    float32 sum -key + gumbel; the r largest are evicted, equal sums taking
    the lower position first. Zero noise evicts the r lowest keys, i.e.
    ``select_keep``.

    Returns the kept slot indices in ascending order (int64).
    """
    pos = np.asarray(pos)[:length]
    key = static_priority(np.asarray(score32, dtype=np.float32)[:length],
                          pos, log_gamma) + np.float32(0.0)
    if n_keep >= length:
        return np.arange(length, dtype=np.int64)
    r = length - n_keep
    cand = np.nonzero(eligible_mask(pos, sinks, window))[0]
    if cand.size < r:
        raise ValueError("not enough eligible entries to evict")
    order = np.lexsort((pos[cand], key[cand]))   # ascending key, then position
    pool = cand[order[:min(2 * r, cand.size)]]
    perturbed = (-key[pool]).astype(np.float32) + \
        np.asarray(gumbel, dtype=np.float32)[pool]
    perturbed = perturbed.astype(np.float32) + np.float32(0.0)
    draw = np.lexsort((pos[pool], -perturbed.astype(np.float64)))
    evicted = np.zeros(length, dtype=bool)
    evicted[pool[draw[:r]]] = True
    return np.nonzero(~evicted)[0].astype(np.int64)


def compaction_sources(keep: np.ndarray) -> np.ndarray:
    """Where each slot of the compacted slice comes from (KVpop Appendix C:
    the decode cache holds only retained entries).

    ``keep`` lists the n_keep kept slots in ascending order. Kept entries in
    slots below n_keep stay where they are; the slots below n_keep that were
    not kept (holes), in ascending order, receive the kept entries from slots
    at or above n_keep, in ascending order. Returns src with
    new[i] = old[src[i]] for i < n_keep.
    """
    keep = np.asarray(keep, dtype=np.int64)
    n_keep = keep.size
    below = keep[keep < n_keep]
    movers = keep[keep >= n_keep]
    holes = np.setdiff1d(np.arange(n_keep, dtype=np.int64), below)
    assert holes.size == movers.size
    src = np.arange(n_keep, dtype=np.int64)
    src[holes] = movers
    return src


def compact_slice(arrays: Sequence[np.ndarray], keep: np.ndarray
                  ) -> List[np.ndarray]:
    """The compacted rows of each array: new row i = old row src[i]
    (``compaction_sources``)."""
    src = compaction_sources(keep)
    return [np.asarray(a)[src].copy() for a in arrays]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def attention_probs(q: np.ndarray, K: np.ndarray):
    """Probabilities of the query heads q [G, d] over the rows K [n, d].

    Logit l = <q, k> / sqrt(d_k) (KVpop Eq. (27)); LSE = log sum exp l
    (Eq. (28)); p = exp(l - LSE) (Eq. (29)). The maximum logit is subtracted
    before exponentiation; it cancels exactly in p and is added back to LSE.
    Returns (p [G, n], lse [G]).
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    d = q.shape[-1]
    logits = (q @ K.T) / np.sqrt(d)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    tot = w.sum(axis=1, keepdims=True)
    p = w / tot
    lse = (m + np.log(tot))[:, 0]
    return p, lse


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Decode attention of G query heads over one KV head's retained rows:
    out = sum_t p_t v_t. Returns (out [G, d], lse [G])."""
    p, lse = attention_probs(q, K)
    return p @ np.asarray(V, np.float64), lse


# ---------------------------------------------------------------------------
# One layer's cache under the policy (incremental form)
# ---------------------------------------------------------------------------

class OracleLayer:
    """The decode-time cache of one attention layer, every (batch, KV head)
    slice holding the same number of entries.

    State per slice: K, V rows (float64 values of the stored dtype), float32
    score and int64 absolute position. New tokens go to the end; evictions
    fill holes from the end (``compaction_sources``), so slot order is not
    position order.
    Scores are computed when a token is appended; the scorer is stateless so
    this equals scoring the buffered tokens at eviction time.
    """

    def __init__(self, K0: np.ndarray, V0: np.ndarray, score0_32: np.ndarray,
                 policy: Policy, group: int):
        policy.check()
        self.policy = policy
        self.group = group
        self.K = np.array(K0, dtype=np.float64)           # [b][H][n][d]
        self.V = np.array(V0, dtype=np.float64)
        self.score = np.array(score0_32, dtype=np.float32)  # [b][H][n]
        b, H, n, _ = self.K.shape
        self.pos = np.broadcast_to(np.arange(n, dtype=np.int64),
                                   (b, H, n)).copy()
        self.newest = n - 1           # P, absolute position of newest token
        self.last_evict_newest = None  # P_e
        self.evictions = 0

    @property
    def n(self) -> int:
        return self.K.shape[2]

    def _evict_to(self, n_keep: int,
                  gumbel: Optional[np.ndarray] = None) -> np.ndarray:
        """Cut every slice to n_keep entries: the deterministic rule, or
        with ``gumbel`` ([b][H][>= n] noise by slot) the stochastic one."""
        b, H = self.K.shape[:2]
        keeps = np.empty((b, H, n_keep), dtype=np.int64)
        srcs = np.empty((b, H, n_keep), dtype=np.int64)
        lg = self.policy.log_gamma
        for bi in range(b):
            for h in range(H):
                lgh = None if lg is None else lg[h]
                if gumbel is None:
                    keeps[bi, h] = select_keep(
                        self.score[bi, h], self.pos[bi, h], self.n, n_keep,
                        self.policy.sinks, self.policy.window, lgh)
                else:
                    keeps[bi, h] = select_keep_stochastic(
                        self.score[bi, h], self.pos[bi, h], self.n, n_keep,
                        self.policy.sinks, self.policy.window,
                        gumbel[bi, h], lgh)
                srcs[bi, h] = compaction_sources(keeps[bi, h])
        idx = srcs[..., None]
        self.K = np.take_along_axis(self.K, idx, axis=2)
        self.V = np.take_along_axis(self.V, idx, axis=2)
        self.score = np.take_along_axis(self.score, srcs, axis=2)
        self.pos = np.take_along_axis(self.pos, srcs, axis=2)
        self.last_evict_newest = self.newest
        self.evictions += 1
        return keeps

    def prefill_compress(self) -> Optional[np.ndarray]:
        """One-shot compression after prefill when n0 > B (reading: compress
        before the first decode step)."""
        if self.n > self.policy.budget:
            return self._evict_to(self.policy.budget)
        return None

    def append(self, k_new: np.ndarray, v_new: np.ndarray,
               score_new_32: np.ndarray) -> None:
        """Append the newest token (k, v [b][H][d], score [b][H])."""
        self.newest += 1
        self.K = np.concatenate([self.K, np.asarray(k_new, np.float64)[:, :, None]], 2)
        self.V = np.concatenate([self.V, np.asarray(v_new, np.float64)[:, :, None]], 2)
        self.score = np.concatenate(
            [self.score, np.asarray(score_new_32, np.float32)[:, :, None]], 2)
        b, H = self.K.shape[:2]
        self.pos = np.concatenate(
            [self.pos, np.full((b, H, 1), self.newest, dtype=np.int64)], 2)

    def set_scores(self, position: int, score_32: np.ndarray) -> None:
        """Give the token at ``position`` its score (score [b][H]): a
        stateful scorer scores a token only when it leaves the window (KVpop
        section 3.3, Eq. 10-11), after the token was appended."""
        hit = self.pos == position
        assert np.all(hit.sum(axis=2) == 1), "token not cached in every slice"
        sc = np.asarray(score_32, np.float32)
        self.score[hit] = np.broadcast_to(sc[:, :, None], hit.shape)[hit]

    def maybe_evict(self, gumbel: Optional[np.ndarray] = None
                    ) -> Optional[np.ndarray]:
        """Evict n - B entries once the cache reaches B + L (with
        ``gumbel``, by ForesightKV's stochastic rule)."""
        p = self.policy
        if self.n >= p.budget + p.evict_len:
            return self._evict_to(p.budget, gumbel)
        return None

    def attend(self, q: np.ndarray):
        """q [b][H*G][d] -> out [b][H*G][d], lse [b][H*G]."""
        b, H = self.K.shape[:2]
        G = self.group
        d = q.shape[-1]
        out = np.empty((b, H * G, d))
        lse = np.empty((b, H * G))
        for bi in range(b):
            for h in range(H):
                o, l_ = decode_attention(q[bi, h * G:(h + 1) * G],
                                         self.K[bi, h], self.V[bi, h])
                out[bi, h * G:(h + 1) * G] = o
                lse[bi, h * G:(h + 1) * G] = l_
        return out, lse

    def step(self, k_new, v_new, score_new_32, q):
        """One decode step: append, evict if due, attend."""
        self.append(k_new, v_new, score_new_32)
        keeps = self.maybe_evict()
        out, lse = self.attend(q)
        return out, lse, keeps

    def state(self) -> dict:
        """A copy of the full decode state (checkpoint)."""
        return {"K": self.K.copy(), "V": self.V.copy(),
                "score": self.score.copy(), "pos": self.pos.copy(),
                "newest": self.newest, "last": self.last_evict_newest,
                "evictions": self.evictions}

    @classmethod
    def from_state(cls, st: dict, policy: Policy, group: int) -> "OracleLayer":
        obj = cls.__new__(cls)
        obj.policy, obj.group = policy, group
        obj.K, obj.V = st["K"].copy(), st["V"].copy()
        obj.score, obj.pos = st["score"].copy(), st["pos"].copy()
        obj.newest, obj.last_evict_newest = st["newest"], st["last"]
        obj.evictions = st["evictions"]
        return obj


# ---------------------------------------------------------------------------
# Closed form of the retained set (second, independent oracle)
# ---------------------------------------------------------------------------

def closed_form_retained(score_by_pos32: np.ndarray, newest: int,
                         last_evict_newest: Optional[int],
                         policy: Policy,
                         log_gamma: Optional[float] = None) -> np.ndarray:
    """Retained positions of one slice after any number of steps, without
    simulating the loop (KVpop Eq. (26) in cache form).

    With a static ranking key (the score, or the static priority of Eq. (20)
    under decay), every evicted token is beaten by k eligible tokens that
    stay eligible, so at the last eviction (newest position P_e) the kept
    long-range tokens are exactly TopK_k(E(P_e)); tokens appended since then
    are all still present. Result: sinks {0..S-1}, the top-k of
    E(P_e) = {S <= t <= P_e - W} by (key desc, position desc), and every
    position in (P_e - W, newest]. ``score_by_pos32`` holds the float32
    score of every position 0..newest. Returns sorted positions.
    """
    S, W, k = policy.sinks, policy.window, policy.k
    if last_evict_newest is None:
        return np.arange(newest + 1, dtype=np.int64)
    pe = last_evict_newest
    elig = np.arange(S, pe - W + 1, dtype=np.int64)
    s = static_priority(np.asarray(score_by_pos32, np.float32)[elig], elig,
                        log_gamma) + np.float32(0.0)
    order = np.lexsort((-elig, -s.astype(np.float64)))  # key desc, pos desc
    top = elig[order[:k]]
    recent = np.arange(max(pe - W + 1, S), newest + 1, dtype=np.int64)
    return np.unique(np.concatenate([np.arange(S, dtype=np.int64), top,
                                     recent]))


# ---------------------------------------------------------------------------
# Cache size per token
# ---------------------------------------------------------------------------

def prefill_ranks(score32: np.ndarray, log_gamma: Optional[float] = None
                  ) -> np.ndarray:
    """rank(t) of every prompt token t = 0..n-1 under the static priority
    (KVpop Appendix C.1; Eq. (20) with decay): rank 0 is the highest
    priority. Order by the float32 key descending, and among equal keys by
    position descending, the reverse of the eviction order of
    ``select_keep`` (equal keys evict the older token first). score32 is
    indexed by position."""
    s = np.asarray(score32, dtype=np.float32)
    n = s.shape[0]
    pos = np.arange(n)
    key = static_priority(s, pos, log_gamma).astype(np.float64) + 0.0
    order = np.lexsort((-pos, -key))  # last key is primary
    rank = np.empty(n, dtype=np.int64)
    rank[order] = np.arange(n)
    return rank


def prefill_cutoffs(rank: np.ndarray, sinks: int, window: int, k: int
                    ) -> np.ndarray:
    """Cutoff rank tau_q for every query position q = 0..n-1 (KVpop
    Appendix C.1-C.2): the rank of the k-th best token of the eligible set
    E(q) = {t : S <= t <= q - W}. Encoded as n when E(q) holds fewer than k
    tokens (every eligible token is kept) and -1 when k = 0 (none is)."""
    rank = np.asarray(rank, dtype=np.int64)
    n = rank.shape[0]
    tau = np.empty(n, dtype=np.int64)
    for q in range(n):
        elig = rank[sinks:max(q - window + 1, sinks)]
        if k == 0:
            tau[q] = -1
        elif elig.shape[0] < k:
            tau[q] = n
        else:
            tau[q] = np.sort(elig)[k - 1]
    return tau


def prefill_mask(rank: np.ndarray, tau: np.ndarray, sinks: int, window: int
                 ) -> np.ndarray:
    """The fixed-budget sparse mask of KVpop Appendix C.1, Eq. (26), over
    causal pairs: M[q, t] = t <= q and (t < S, or q - t < W, or t in E(q)
    with rank(t) <= tau_q). Returns bool [n][n]."""
    n = np.asarray(rank).shape[0]
    q = np.arange(n)[:, None]
    t = np.arange(n)[None, :]
    sink = t < sinks
    recent = (q - t) < window
    elig = (t >= sinks) & (t <= q - window)
    top = elig & (np.asarray(rank)[None, :] <= np.asarray(tau)[:, None])
    return (t <= q) & (sink | recent | top)


def prefill_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                      masks: np.ndarray, group: int):
    """Masked attention over the prompt (KVpop Appendix C, Eq. (26) applied
    inside the attention of Appendix D.1, Eq. (27)-(29)) for one sequence:
    Q [H*G][n][d], K and V [H][n][d], masks [H][n][n] (per KV head; query
    head j reads KV head floor(j / G)). Returns out [H*G][n][d] and the
    natural-log normaliser lse [H*G][n]; a query with no kept key gets
    out = 0 and lse = -inf."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, n, d = Q.shape
    out = np.zeros((hq, n, d))
    lse = np.full((hq, n), -np.inf)
    for j in range(hq):
        h = j // group
        z = (Q[j] @ K[h].T) / np.sqrt(d)
        z = np.where(masks[h], z, -np.inf)
        m = z.max(axis=1)
        ok = np.isfinite(m)
        e = np.exp(z[ok] - m[ok, None])
        ssum = e.sum(axis=1)
        out[j, ok] = (e / ssum[:, None]) @ V[h]
        lse[j, ok] = m[ok] + np.log(ssum)
    return out, lse


def cache_bytes_per_token(layers: int, n_kv: int, head_dim: int,
                          elem_bytes: int) -> int:
    """A GQA layer stores 2 * n_kv * d_h scalars per token (KV-Kaizen,
    section 2.1 "Background and notation"); summed over layers."""
    return layers * 2 * n_kv * head_dim * elem_bytes
