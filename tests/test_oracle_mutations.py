"""Planted mistakes in (copies of) the oracle must fail its pins.

Each mutant below is the oracle function with one plausible mistake (a
dropped term, a swapped operand, a reversed tie-break, an off-by-one). The
pin checks from ``test_oracle_pins`` are run against it and must fail, which
shows that the pins constrain every part of the oracle. Runs on the CPU.
"""
import numpy as np
import pytest

import oracle as O
import test_oracle_pins as P


def _fails(check, impl):
    with pytest.raises(AssertionError):
        check(impl)


# --- scorer mutants --------------------------------------------------------

def mlp_vk_order(k, v, w1, b1, w2, b2, act="relu"):
    return O.mlp_score(v, k, w1, b1, w2, b2, act)


def mlp_no_b1(k, v, w1, b1, w2, b2, act="relu"):
    return O.mlp_score(k, v, w1, np.zeros_like(np.asarray(b1, float)), w2,
                       b2, act)


def mlp_no_activation(k, v, w1, b1, w2, b2, act="relu"):
    x = np.concatenate([k, v], axis=-1)
    return (x @ np.asarray(w1).T + b1) @ np.asarray(w2) + b2


def gate_linear(hidden, w, b=0.0):
    return np.asarray(hidden) @ np.asarray(w) + b


@pytest.mark.parametrize("mutant", [mlp_vk_order, mlp_no_b1,
                                    mlp_no_activation])
def test_mlp_mutants_fail_hand_case(mutant):
    _fails(P.check_mlp_hand, mutant)


def test_mlp_no_activation_fails_one_hot():
    _fails(P.check_mlp_one_hot, mlp_no_activation)


def test_gate_without_sigmoid_fails():
    _fails(P.check_gate, gate_linear)


# --- selection mutants -----------------------------------------------------

def select_newest_first_on_ties(score32, pos, length, n_keep, sinks, window):
    if n_keep >= length:
        return np.arange(length)
    r = length - n_keep
    pos = np.asarray(pos)[:length]
    cand = np.nonzero(O.eligible_mask(pos, sinks, window))[0]
    order = np.lexsort((-pos[cand], np.asarray(score32)[cand]))
    ev = np.zeros(length, bool)
    ev[cand[order[:r]]] = True
    return np.nonzero(~ev)[0]


def select_by_slot_ranges(score32, pos, length, n_keep, sinks, window):
    """Protects slots [0, S) and [len - W, len) instead of positions."""
    if n_keep >= length:
        return np.arange(length)
    r = length - n_keep
    cand = np.arange(sinks, length - window)
    order = np.lexsort((np.asarray(pos)[cand], np.asarray(score32)[cand]))
    ev = np.zeros(length, bool)
    ev[cand[order[:r]]] = True
    return np.nonzero(~ev)[0]


def select_window_off_by_one(score32, pos, length, n_keep, sinks, window):
    return O.select_keep(score32, pos, length, n_keep, sinks,
                         max(window - 1, 0))


def select_evicts_highest(score32, pos, length, n_keep, sinks, window):
    return O.select_keep(-np.asarray(score32), pos, length, n_keep, sinks,
                         window)


@pytest.mark.parametrize("mutant", [select_newest_first_on_ties,
                                    select_by_slot_ranges,
                                    select_window_off_by_one,
                                    select_evicts_highest])
def test_select_mutants_fail(mutant):
    failed = 0
    for check in (P.check_select_hand, P.check_select_brute_force):
        try:
            check(mutant)
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1


def closed_form_oldest_kept(score_by_pos32, newest, last, policy):
    S, W, k = policy.sinks, policy.window, policy.k
    if last is None:
        return np.arange(newest + 1)
    elig = np.arange(S, last - W + 1)
    s = np.asarray(score_by_pos32, np.float32)[elig]
    order = np.lexsort((elig, -s.astype(np.float64)))   # pos ascending: wrong
    top = elig[order[:k]]
    recent = np.arange(max(last - W + 1, S), newest + 1)
    return np.unique(np.concatenate([np.arange(S), top, recent]))


def sources_order_preserving(keep):
    return np.asarray(keep)


def sources_movers_reversed(keep):
    keep = np.asarray(keep)
    n = keep.size
    src = np.arange(n)
    holes = np.setdiff1d(np.arange(n), keep[keep < n])
    src[holes] = keep[keep >= n][::-1]
    return src


@pytest.mark.parametrize("mutant", [sources_order_preserving,
                                    sources_movers_reversed])
def test_compaction_mutants_fail(mutant):
    _fails(P.check_compaction, mutant)


def test_closed_form_mutant_fails():
    _fails(P.check_incremental_equals_closed_form, closed_form_oldest_kept)


# --- attention mutants -----------------------------------------------------

def attn_no_scale(q, K, V):
    d = q.shape[-1]
    return O.decode_attention(np.asarray(q) * np.sqrt(d), K, V)


def attn_k_v_swapped(q, K, V):
    return O.decode_attention(q, V, K)


def attn_unnormalised_lse(q, K, V):
    out, lse = O.decode_attention(q, K, V)
    logits = np.asarray(q) @ np.asarray(K).T / np.sqrt(q.shape[-1])
    return out, logits.max(axis=1)


@pytest.mark.parametrize("mutant", [attn_no_scale, attn_k_v_swapped,
                                    attn_unnormalised_lse])
def test_attention_mutants_fail(mutant):
    _fails(P.check_attention_hand, mutant)
    _fails(P.check_attention_vs_torch_sdpa, mutant)


def select_decay_wrong_sign(score32, pos, length, n_keep, sinks, window,
                            log_gamma=None):
    """Adds t log(gamma) instead of subtracting it (favours old tokens)."""
    lg = None if log_gamma is None else -log_gamma
    return O.select_keep(score32, pos, length, n_keep, sinks, window, lg)


def select_decay_ignored(score32, pos, length, n_keep, sinks, window,
                         log_gamma=None):
    return O.select_keep(score32, pos, length, n_keep, sinks, window)


@pytest.mark.parametrize("mutant", [select_decay_wrong_sign,
                                    select_decay_ignored])
def test_decay_mutants_fail(mutant):
    _fails(P.check_decay_ranking, mutant)


# --- mLSTM scorer mutants --------------------------------------------------

class MlstmNoForget(O.MlstmScorer):
    """Ignores the forget gate (f = 1)."""

    def push(self, x):
        self.q += 1
        qf, kf, vf, ig, fg = O.mlstm_features(x, self.w)
        self.C = self.C + ig * np.outer(kf, vf)
        self.z = self.z + ig * kf
        self.qf[self.q] = qf
        u = self.q - self.window
        if u < 0:
            return None
        return u, O.mlstm_readout(self.qf.pop(u), self.C, self.z, self.w)


class MlstmReadBeforeWrite(O.MlstmScorer):
    """Reads token u out of the state before absorbing token q."""

    def push(self, x):
        self.q += 1
        qf, kf, vf, ig, fg = O.mlstm_features(x, self.w)
        self.qf[self.q] = qf
        u = self.q - self.window
        res = None
        if u >= 0 and self.q > 0:
            res = (u, O.mlstm_readout(self.qf.pop(u), self.C, self.z, self.w))
        self.C = fg * self.C + ig * np.outer(kf, vf)
        self.z = fg * self.z + ig * kf
        if u >= 0 and res is None:
            res = (u, O.mlstm_readout(self.qf.pop(u), self.C, self.z, self.w))
        return res


class MlstmNoNormaliser(O.MlstmScorer):
    """Reads h = q~ . C without dividing by the normaliser q~ . z."""

    def push(self, x):
        self.q += 1
        qf, kf, vf, ig, fg = O.mlstm_features(x, self.w)
        self.C = fg * self.C + ig * np.outer(kf, vf)
        self.z = fg * self.z + ig * kf
        self.qf[self.q] = qf
        u = self.q - self.window
        if u < 0:
            return None
        h = self.qf.pop(u) @ self.C
        return u, float(self.w.a @ (h / (1.0 + np.exp(-h))) + self.w.b)


@pytest.mark.parametrize("mutant", [MlstmNoForget, MlstmReadBeforeWrite,
                                    MlstmNoNormaliser])
def test_mlstm_mutants_fail(mutant):
    failed = 0
    for check in (P.check_mlstm_hand, P.check_mlstm_recurrent_equals_parallel):
        try:
            check(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1


# --- prefill selection mutants ----------------------------------------------

def ranks_ties_older_first(s32, log_gamma=None):
    """Equal keys ranked older-first (the wrong tie order)."""
    n = s32.shape[0]
    key = O.static_priority(s32, np.arange(n), log_gamma).astype(np.float64) + 0.0
    order = np.lexsort((np.arange(n), -key))
    r = np.empty(n, dtype=np.int64)
    r[order] = np.arange(n)
    return r


def cutoffs_off_by_one(rank, sinks, window, k):
    """The (k+1)-th best instead of the k-th."""
    return O.prefill_cutoffs(rank, sinks, window, k + 1)


def mask_window_inclusive(rank, tau, sinks, window):
    """Window read as q - t <= W."""
    return O.prefill_mask(rank, tau, sinks, window + 1)


def mask_without_sinks(rank, tau, sinks, window):
    n = np.asarray(rank).shape[0]
    M = O.prefill_mask(rank, tau, sinks, window)
    elig = np.arange(n)[None, :] >= sinks
    return M & (elig | (np.arange(n)[:, None] - np.arange(n)[None, :] < window))


@pytest.mark.parametrize("fns", [
    (ranks_ties_older_first, O.prefill_cutoffs, O.prefill_mask),
    (O.prefill_ranks, cutoffs_off_by_one, O.prefill_mask),
    (O.prefill_ranks, O.prefill_cutoffs, mask_window_inclusive),
    (O.prefill_ranks, O.prefill_cutoffs, mask_without_sinks),
], ids=["rank-ties", "cutoff-k+1", "window-inclusive", "no-sinks"])
def test_prefill_mutants_fail(fns):
    failed = 0
    for check in (P.check_prefill_hand, P.check_prefill_mask_equals_decode_loop):
        try:
            check(*fns)
        except AssertionError:
            failed += 1
    assert failed >= 1


# --- sink-attention gate mutants --------------------------------------------

def sink_gate_mean(hidden, w):
    """Mean over the query heads instead of the maximum."""
    G = np.asarray(w.wq).shape[1]
    total = 0.0
    for g in range(G):
        wg = O.SinkGateWeights(w.wk, np.asarray(w.wq)[:, g:g + 1], w.gk, w.gq,
                               w.sinks, np.asarray(w.b)[:, g:g + 1], w.eps)
        total = total + O.sink_gate_score(hidden, wg)
    return total / G


def sink_gate_no_own_term(hidden, w):
    """exp(a) / (sum_r exp(c_r) + b): the token's term left out of the
    denominator."""
    g = O.sink_gate_score(hidden, w)
    return g / (1.0 - g)


def sink_gate_unscaled(hidden, w):
    """Logits without the 1/sqrt(D') scale."""
    dp = np.asarray(w.wq).shape[2]
    return O.sink_gate_score(hidden, O.SinkGateWeights(
        w.wk, np.asarray(w.wq) * np.sqrt(dp) ** 0, w.gk,
        np.asarray(w.gq) * np.sqrt(dp), w.sinks, w.b, w.eps))


@pytest.mark.parametrize("fn", [sink_gate_mean, sink_gate_no_own_term,
                                sink_gate_unscaled],
                         ids=["mean", "no-own-term", "unscaled"])
def test_sink_gate_mutants_fail(fn):
    failed = 0
    for check in (P.check_sink_gate_hand,
                  P.check_sink_gate_without_denominator_is_sigmoid,
                  P.check_sink_gate_sinks_equal_to_key):
        try:
            check(fn)
        except AssertionError:
            failed += 1
    assert failed >= 1


# --- stochastic eviction mutants ---------------------------------------------

def _stoch(score32, pos, length, n_keep, sinks, window, gumbel, log_gamma=None,
           pool_mult=2, sign=-1.0, newer_first=False):
    pos = np.asarray(pos)[:length]
    key = O.static_priority(np.asarray(score32, np.float32)[:length], pos,
                            log_gamma)
    if n_keep >= length:
        return np.arange(length)
    r = length - n_keep
    cand = np.nonzero(O.eligible_mask(pos, sinks, window))[0]
    order = np.lexsort((pos[cand], key[cand]))
    pool = cand[order[:min(pool_mult * r, cand.size)]]
    pert = (np.float32(sign) * key[pool]).astype(np.float32) + \
        np.asarray(gumbel, np.float32)[pool]
    tie = -pos[pool] if newer_first else pos[pool]
    draw = np.lexsort((tie, -pert.astype(np.float64)))
    ev = np.zeros(length, bool)
    ev[pool[draw[:r]]] = True
    return np.nonzero(~ev)[0]


def stoch_greedy_pool(*a, **k):
    """Pool of r: plain greedy eviction, no sampling."""
    return _stoch(*a, pool_mult=1, **k)


def stoch_all_candidates(*a, **k):
    """Draws over every candidate instead of the 2r lowest."""
    return _stoch(*a, pool_mult=10 ** 9, **k)


def stoch_sign_flipped(*a, **k):
    """Weights exp(+score): the highest-scoring pool entries go first."""
    return _stoch(*a, sign=1.0, **k)


def stoch_ties_newer_first(*a, **k):
    """Equal perturbed sums evict the newer token first."""
    return _stoch(*a, newer_first=True, **k)


def test_stochastic_reference_mutant_passes():
    """The helper with the oracle's settings passes every check (so the
    mutants below fail for their planted change alone)."""
    for check in (P.check_stochastic_zero_noise_is_greedy,
                  P.check_stochastic_pool, P.check_stochastic_hand):
        check(_stoch)


@pytest.mark.parametrize("fn", [stoch_greedy_pool, stoch_all_candidates,
                                stoch_sign_flipped, stoch_ties_newer_first],
                         ids=["greedy-pool", "all-candidates", "sign-flipped",
                              "ties-newer-first"])
def test_stochastic_mutants_fail(fn):
    failed = 0
    for check in (P.check_stochastic_zero_noise_is_greedy,
                  P.check_stochastic_pool, P.check_stochastic_hand,
                  P.check_stochastic_distribution):
        try:
            check(fn)
        except AssertionError:
            failed += 1
    assert failed >= 1
