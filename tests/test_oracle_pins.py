"""Pins of the float64 oracle to facts other than its own formulas.

Each check below compares the oracle with a hand-derived closed form, a
library routine (numpy/scipy/torch on the CPU), brute force on tiny inputs,
or an invariant the pages fix. The checks are written as functions of the
implementation so that ``test_oracle_mutations.py`` can show that a planted
mistake in the oracle makes them fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Scorer pins
# ---------------------------------------------------------------------------

def check_mlp_hand(mlp_score):
    g = golden()["mlp_relu"]
    s = mlp_score(np.array(g["k"]), np.array(g["v"]), np.array(g["w1"]),
                  np.array(g["b1"]), np.array(g["w2"]), g["b2"], "relu")
    assert s == pytest.approx(g["expected"], abs=1e-15)


def check_mlp_silu(mlp_score):
    g = golden()["mlp_relu"]
    a = np.array([1.0, -1.0, 2.5])          # pre-activations, by hand
    silu = a * scipy.special.expit(a)       # library sigmoid
    expected = float(np.dot(np.array(g["w2"]), silu) + g["b2"])
    s = mlp_score(np.array(g["k"]), np.array(g["v"]), np.array(g["w1"]),
                  np.array(g["b1"]), np.array(g["w2"]), g["b2"], "silu")
    assert s == pytest.approx(expected, rel=1e-14)


def check_mlp_one_hot(mlp_score):
    # One-hot first layer + ReLU + unit second layer returns relu(x_i).
    rng = np.random.default_rng(3)
    d, hid = 8, 16
    k = rng.standard_normal((50, d))
    v = rng.standard_normal((50, d))
    x = np.concatenate([k, v], axis=1)
    for i in (0, 3, d, 2 * d - 1):
        w1 = np.zeros((hid, 2 * d))
        w1[5, i] = 1.0
        w2 = np.zeros(hid)
        w2[5] = 1.0
        s = mlp_score(k, v, w1, np.zeros(hid), w2, 0.0, "relu")
        np.testing.assert_array_equal(s, np.maximum(x[:, i], 0.0))


def check_gate(gate_score):
    g = golden()["gate"]
    assert gate_score(np.array(g["hidden"]), np.array(g["w"]), g["b"]) == \
        pytest.approx(g["expected"], abs=1e-15)
    rng = np.random.default_rng(4)
    h = rng.standard_normal((40, 64))
    w = rng.standard_normal(64) / 8
    np.testing.assert_allclose(gate_score(h, w, 0.3),
                               scipy.special.expit(h @ w + 0.3), rtol=1e-14)


def test_mlp_hand_case():
    check_mlp_hand(O.mlp_score)


def test_mlp_silu_vs_library_sigmoid():
    check_mlp_silu(O.mlp_score)


def test_mlp_one_hot_is_relu_of_input():
    check_mlp_one_hot(O.mlp_score)


def test_gate_hand_case_and_expit():
    check_gate(O.gate_score)


def test_score_to_f32_canonical_zero_and_rounding():
    s = O.score_to_f32(np.array([-0.0, 0.0, 1.0 / 3.0]))
    assert not np.signbit(s[0])
    assert s[2] == np.float32(1.0 / 3.0)
    with pytest.raises(ValueError):
        O.score_to_f32(np.array([np.nan]))


# ---------------------------------------------------------------------------
# Selection pins
# ---------------------------------------------------------------------------

def brute_force_keep(scores, pos, length, n_keep, S, W):
    """Rank every candidate by counting how many candidates precede it in
    (score, position) order; the r lowest ranks are evicted. Candidates are
    the entries whose position t satisfies S <= t <= P - W (P the newest
    position present)."""
    if n_keep >= length:
        return list(range(length))
    r = length - n_keep
    P = max(pos[:length])
    cands = [u for u in range(length) if S <= pos[u] <= P - W]
    keep = []
    for t in range(length):
        if t not in cands:
            keep.append(t)
            continue
        rank = sum(1 for u in cands
                   if (scores[u] < scores[t]) or
                   (scores[u] == scores[t] and pos[u] < pos[t]))
        if rank >= r:
            keep.append(t)
    return keep


def check_select_hand(select_keep):
    g = golden()["selection"]
    sc = np.array(g["scores"], dtype=np.float32)
    keep = select_keep(sc, np.arange(len(sc)), g["length"], g["n_keep"],
                       g["sinks"], g["window"])
    assert list(keep) == g["expected_keep"]


def check_select_brute_force(select_keep):
    alphabet = np.array([0.5, 1.0, 2.0], dtype=np.float32)
    rng = np.random.default_rng(6)
    for S, W in ((0, 0), (1, 2), (2, 1)):
        for m in range(0, 6):
            length = S + W + m
            for pattern in itertools.product(range(3), repeat=length):
                sc = alphabet[list(pattern)]
                # positions 0..length-1 in slot order, and shuffled (a cache
                # whose evictions filled holes from the end)
                for pos in (np.arange(length), rng.permutation(length)):
                    for r in range(0, m + 1):
                        n_keep = length - r
                        got = list(select_keep(sc, pos, length, n_keep, S, W))
                        assert got == brute_force_keep(sc, pos, length,
                                                       n_keep, S, W)


def test_select_hand_case():
    check_select_hand(O.select_keep)


def test_select_matches_brute_force_all_tie_patterns():
    check_select_brute_force(O.select_keep)


def test_select_random_matches_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(200):
        S, W = rng.integers(0, 4), rng.integers(0, 6)
        m = rng.integers(0, 25)
        length = S + W + m
        sc = rng.integers(0, 5, size=length).astype(np.float32) * 0.25
        r = rng.integers(0, m + 1)
        pos = rng.permutation(length) + 0
        got = list(O.select_keep(sc, pos, length, length - r, S, W))
        assert got == brute_force_keep(sc, pos, length, length - r, S, W)


def test_select_k_zero_keeps_sinks_and_window_only():
    rng = np.random.default_rng(8)
    sc = rng.standard_normal(40).astype(np.float32)
    keep = O.select_keep(sc, np.arange(40), 40, 10, 4, 6)
    assert list(keep) == [0, 1, 2, 3] + list(range(34, 40))


def test_select_budget_above_length_keeps_all():
    sc = np.ones(30, dtype=np.float32)
    assert list(O.select_keep(sc, np.arange(30), 30, 64, 4, 8)) == \
        list(range(30))


def test_constant_scores_give_streaming_llm():
    """Constant scores reduce the policy to sinks + most recent tokens
    (StreamingLLM, KVpop section 2 'Heuristic eviction methods')."""
    pol = O.Policy(budget=24, sinks=3, window=5, evict_len=4)
    rng = np.random.default_rng(9)
    n0, d = 40, 8
    K0 = rng.standard_normal((1, 1, n0, d))
    lay = O.OracleLayer(K0, K0, np.zeros((1, 1, n0), np.float32), pol, 1)
    lay.prefill_compress()
    expected = list(range(3)) + list(range(n0 - 21, n0))
    assert sorted(lay.pos[0, 0]) == expected
    for _ in range(13):
        kn = rng.standard_normal((1, 1, d))
        lay.append(kn, kn, np.zeros((1, 1), np.float32))
        if lay.maybe_evict() is not None:
            P = lay.newest
            assert sorted(lay.pos[0, 0]) == list(range(3)) + \
                list(range(P - 20, P + 1))


def brute_force_sources(keep, n_keep):
    """Hole filling written out slot by slot: walk the slots below n_keep in
    order; a kept slot stays, a hole takes the next kept slot at or above
    n_keep (in order)."""
    kept = set(int(x) for x in keep)
    movers = [int(x) for x in keep if x >= n_keep]
    src, nxt = [], 0
    for i in range(n_keep):
        if i in kept:
            src.append(i)
        else:
            src.append(movers[nxt])
            nxt += 1
    assert nxt == len(movers)
    return src


def check_compaction(compaction_sources):
    rng = np.random.default_rng(21)
    for _ in range(300):
        length = int(rng.integers(1, 40))
        n_keep = int(rng.integers(0, length + 1))
        keep = np.sort(rng.choice(length, n_keep, replace=False))
        src = list(compaction_sources(keep))
        assert src == brute_force_sources(keep, n_keep)
        # the compacted slice holds exactly the kept entries ...
        assert sorted(src) == list(keep)
        # ... kept entries below n_keep never move, and only the kept
        # entries at or above n_keep are moved
        for i, j in enumerate(src):
            if j != i:
                assert j >= n_keep and i not in set(keep.tolist())
    # hand case: slots 0..7 cut to 5, keep {0, 2, 5, 6, 7}: holes 1, 3, 4
    # take 5, 6, 7 in order
    assert list(compaction_sources(np.array([0, 2, 5, 6, 7]))) == \
        [0, 5, 2, 6, 7]


def test_compaction_hole_filling():
    check_compaction(O.compaction_sources)


def test_compact_slice_moves_rows_bitwise():
    rng = np.random.default_rng(22)
    K = rng.standard_normal((12, 3))
    pos = np.arange(12) * 7
    keep = np.array([0, 1, 4, 8, 9, 11])
    K2, pos2 = O.compact_slice([K, pos], keep)
    src = [0, 1, 8, 9, 4, 11]   # holes 2, 3, 5 take 8, 9, 11
    np.testing.assert_array_equal(K2, K[src])
    np.testing.assert_array_equal(pos2, pos[src])


# ---------------------------------------------------------------------------
# Incremental loop vs closed form; invariants
# ---------------------------------------------------------------------------

def run_incremental(policy, n0, steps, scores_by_pos, seed=0, d=4):
    """Drive OracleLayer with a given score per position (1 slice)."""
    rng = np.random.default_rng(seed)
    K0 = rng.standard_normal((1, 1, n0, d))
    lay = O.OracleLayer(K0, K0, scores_by_pos[None, None, :n0], policy, 1)
    history = []
    lay.prefill_compress()
    history.append((lay.newest, lay.last_evict_newest,
                    np.sort(lay.pos[0, 0])))
    for i in range(steps):
        kn = rng.standard_normal((1, 1, d))
        lay.append(kn, kn, scores_by_pos[n0 + i].reshape(1, 1))
        lay.maybe_evict()
        history.append((lay.newest, lay.last_evict_newest,
                        np.sort(lay.pos[0, 0])))
    return history


def check_incremental_equals_closed_form(closed_form):
    rng = np.random.default_rng(11)
    for (B, S, W, L, n0) in ((20, 2, 4, 1, 30), (20, 2, 4, 5, 30),
                             (16, 0, 3, 3, 10), (12, 3, 9, 2, 50),
                             (32, 4, 8, 8, 31)):
        pol = O.Policy(B, S, W, L)
        steps = 60
        for mode in ("cont", "ties"):
            if mode == "cont":
                sc = rng.standard_normal(n0 + steps).astype(np.float32)
            else:
                sc = rng.integers(0, 3, n0 + steps).astype(np.float32)
            for newest, pe, kept in run_incremental(pol, n0, steps, sc):
                cf = closed_form(sc[:newest + 1], newest, pe, pol)
                np.testing.assert_array_equal(kept, cf)


def test_incremental_loop_equals_closed_form():
    check_incremental_equals_closed_form(O.closed_form_retained)


def test_invariants_over_config1_shape():
    """Sinks and window are never evicted, count == B after every eviction,
    positions distinct (KVpop Eq. (1), Eq. (26))."""
    w = syn.workload(1)
    pol = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    rng = np.random.default_rng(12)
    n0 = w.n0
    sc = rng.standard_normal(n0 + w.steps).astype(np.float32)
    for newest, pe, kept in run_incremental(pol, n0, w.steps, sc):
        assert np.all(np.diff(kept) > 0)           # sorted, hence distinct
        assert set(range(w.sinks)) <= set(kept)
        assert set(range(newest - w.window + 1, newest + 1)) <= set(kept)
        assert len(kept) <= w.budget + w.evict_len - 1
        if pe == newest:
            assert len(kept) == w.budget


def test_checkpoint_resume_is_bitwise_identical():
    pol = O.Policy(24, 2, 6, 4)
    rng = np.random.default_rng(13)
    n0, d, b, H, G = 40, 8, 2, 2, 2
    K0 = rng.standard_normal((b, H, n0, d))
    V0 = rng.standard_normal((b, H, n0, d))
    s0 = rng.standard_normal((b, H, n0)).astype(np.float32)
    steps = [(rng.standard_normal((b, H, d)), rng.standard_normal((b, H, d)),
              rng.standard_normal((b, H)).astype(np.float32),
              rng.standard_normal((b, H * G, d))) for _ in range(20)]
    a = O.OracleLayer(K0, V0, s0, pol, G)
    a.prefill_compress()
    outs_a = [a.step(*s)[:2] for s in steps]
    c = O.OracleLayer(K0, V0, s0, pol, G)
    c.prefill_compress()
    outs_c = [c.step(*s)[:2] for s in steps[:7]]
    c2 = O.OracleLayer.from_state(c.state(), pol, G)
    outs_c += [c2.step(*s)[:2] for s in steps[7:]]
    for (oa, la), (oc, lc) in zip(outs_a, outs_c):
        np.testing.assert_array_equal(oa, oc)
        np.testing.assert_array_equal(la, lc)


# ---------------------------------------------------------------------------
# Attention pins
# ---------------------------------------------------------------------------

def check_attention_hand(decode_attention):
    g = golden()["attention_two_rows"]
    out, lse = decode_attention(np.array(g["q"]), np.array(g["K"]),
                                np.array(g["V"]))
    e = math.e
    np.testing.assert_allclose(out[0], [e / (e + 1), 1 / (e + 1), 0, 0],
                               rtol=1e-15, atol=1e-16)
    assert lse[0] == pytest.approx(math.log(e + 1), rel=1e-15)


def check_attention_vs_torch_sdpa(decode_attention):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(14)
    G, n, d = 4, 37, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d)) * 2
    V = rng.standard_normal((n, d))
    out, lse = decode_attention(q, K, V)
    tq = torch.from_numpy(q)[None, :, None, :]           # [1, G, 1, d]
    tk = torch.from_numpy(K)[None, None].expand(1, G, n, d).contiguous()
    tv = torch.from_numpy(V)[None, None].expand(1, G, n, d).contiguous()
    ref = F.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    logits = q @ K.T / np.sqrt(d)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(logits, axis=1),
                               rtol=1e-13)


def test_attention_hand_case():
    check_attention_hand(O.decode_attention)


def test_attention_equals_torch_sdpa_float64_and_logsumexp():
    check_attention_vs_torch_sdpa(O.decode_attention)


def test_attention_probabilities_sum_to_one():
    rng = np.random.default_rng(15)
    for n in (1, 2, 17, 300):
        p, _ = O.attention_probs(rng.standard_normal((5, 32)) * 3,
                                 rng.standard_normal((n, 32)) * 3)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        assert np.all(p >= 0)


def test_attention_single_row_and_identical_keys():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    out, lse = O.decode_attention(q, k, v)
    np.testing.assert_array_equal(out, np.repeat(v, 3, axis=0))
    np.testing.assert_allclose(lse, (q @ k.T)[:, 0] / np.sqrt(8), rtol=1e-15)
    K = np.repeat(k, 10, axis=0)
    V = rng.standard_normal((10, 8))
    out, _ = O.decode_attention(q, K, V)
    np.testing.assert_allclose(out, np.repeat(V.mean(0, keepdims=True), 3, 0),
                               rtol=1e-13, atol=1e-15)


def test_attention_permutation_invariant():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((50, 16))
    V = rng.standard_normal((50, 16))
    perm = rng.permutation(50)
    o1, l1 = O.decode_attention(q, K, V)
    o2, l2 = O.decode_attention(q, K[perm], V[perm])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_budget_above_length_equals_dense_attention_every_step():
    """With B at or above the context length nothing is evicted and each
    step's output equals dense attention over the whole history."""
    rng = np.random.default_rng(18)
    b, H, G, d, n0 = 1, 2, 3, 8, 12
    pol = O.Policy(budget=64, sinks=2, window=4, evict_len=8)
    K = rng.standard_normal((b, H, n0, d))
    V = rng.standard_normal((b, H, n0, d))
    lay = O.OracleLayer(K, V, rng.standard_normal((b, H, n0)).astype(
        np.float32), pol, G)
    assert lay.prefill_compress() is None
    allK, allV = K.copy(), V.copy()
    for _ in range(40):
        kn, vn = rng.standard_normal((b, H, d)), rng.standard_normal((b, H, d))
        q = rng.standard_normal((b, H * G, d))
        out, lse, keeps = lay.step(kn, vn, rng.standard_normal((b, H)).astype(
            np.float32), q)
        allK = np.concatenate([allK, kn[:, :, None]], 2)
        allV = np.concatenate([allV, vn[:, :, None]], 2)
        if lay.n <= pol.budget + pol.evict_len - 1 and keeps is None:
            for h in range(H):
                for g in range(G):
                    logits = allK[0, h] @ q[0, h * G + g] / np.sqrt(d)
                    p = scipy.special.softmax(logits)
                    np.testing.assert_allclose(out[0, h * G + g],
                                               p @ allV[0, h], rtol=1e-12,
                                               atol=1e-14)


# ---------------------------------------------------------------------------
# Byte accounting pins (numbers printed on the pages)
# ---------------------------------------------------------------------------

def test_qwen3_4b_cache_is_4_5_gb_at_32k():
    """ForesightKV summary, 'Main findings': 4.5 GB bf16 cache for one
    Qwen3-4B instance at 32K tokens."""
    per_tok = O.cache_bytes_per_token(36, 8, 128, 2)
    assert per_tok == 144 * 1024
    assert per_tok * 32768 == int(4.5 * 2 ** 30)


def test_qwen25_14b_cache_is_192_kib_per_token():
    """KV-Kaizen section 1: 192 KiB per token; 32 sequences of 8k tokens
    fill 48 GiB."""
    per_tok = O.cache_bytes_per_token(48, 8, 128, 2)
    assert per_tok == 192 * 1024
    assert 32 * 8192 * per_tok == 48 * 2 ** 30


# ---------------------------------------------------------------------------
# Input generator pins
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(19)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000)
         ).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # exact ties
    ours = syn.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy(
        ).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_is_deterministic_and_keyed():
    w = syn.workload(2, batch=2, n0=64)
    a = syn.initial_context(w, 0, 0)
    b = syn.initial_context(w, 0, 0)
    c = syn.initial_context(w, 1, 0)
    np.testing.assert_array_equal(a["k0"].bits, b["k0"].bits)
    assert not np.array_equal(a["k0"].bits, c["k0"].bits)
    s0 = syn.step_inputs(w, 0, 0, 0)
    s1 = syn.step_inputs(w, 0, 0, 1)
    assert not np.array_equal(s0["q"].bits, s1["q"].bits)
    assert a["k0"].shape == (2, 8, 64, 128)


# ---------------------------------------------------------------------------
# Temporal decay (KVpop Eq. (5), Appendix B.3 Eq. (18)-(20), n = 1)
# ---------------------------------------------------------------------------

def brute_force_keep_effective(scores, pos, length, n_keep, S, W, log_gamma):
    """Evict the r eligible tokens with the lowest effective score at the
    newest position q = P, r + (q - t) log(gamma), computed in float64 (ties
    by older position first)."""
    if n_keep >= length:
        return list(range(length))
    r = length - n_keep
    q = max(pos[:length])
    cands = [u for u in range(length) if S <= pos[u] <= q - W]
    eff = {u: float(scores[u]) + (q - pos[u]) * log_gamma for u in cands}
    order = sorted(cands, key=lambda u: (eff[u], pos[u]))
    evicted = set(order[:r])
    return [t for t in range(length) if t not in evicted]


def check_decay_ranking(select_keep):
    """Eq. (19)-(20): at a fixed query position the effective-score ranking
    equals the static-priority ranking (checked where the float64 effective
    scores are far apart compared with float32 rounding)."""
    rng = np.random.default_rng(31)
    checked = 0
    for _ in range(400):
        S, W = int(rng.integers(0, 4)), int(rng.integers(0, 6))
        m = int(rng.integers(1, 30))
        length = S + W + m
        pos = rng.permutation(length) + 0
        sc = rng.standard_normal(length).astype(np.float32)
        lg = float(np.log(rng.uniform(0.5, 0.99)))
        q = pos.max()
        eff = np.sort(sc.astype(np.float64) + (q - pos) * lg)
        if np.min(np.diff(eff)) < 1e-4:
            continue
        r = int(rng.integers(0, m + 1))
        got = list(select_keep(sc, pos, length, length - r, S, W, lg))
        assert got == brute_force_keep_effective(sc, pos, length, length - r,
                                                 S, W, lg)
        checked += 1
    assert checked > 200


def test_decay_ranking_equals_effective_score_ranking():
    check_decay_ranking(O.select_keep)


def test_decay_hand_case():
    # positions 0..5, S = 1, W = 1: candidates are positions 1..4 with
    # scores 0.6, 0.9, 0.9, 0.45. With log(gamma) = -0.1 the static
    # priorities r - t log(gamma) are 0.7, 1.1, 1.2, 0.85, so evicting one
    # drops the old t = 1; without decay the lowest score, t = 4, goes.
    sc = np.array([9.0, 0.6, 0.9, 0.9, 0.45, 9.0], np.float32)
    keep = O.select_keep(sc, np.arange(6), 6, 5, 1, 1, -0.1)
    assert list(keep) == [0, 2, 3, 4, 5]
    assert list(O.select_keep(sc, np.arange(6), 6, 5, 1, 1)) == \
        [0, 1, 2, 3, 5]


def test_decay_zero_is_no_decay_and_prefers_recent():
    rng = np.random.default_rng(32)
    sc = rng.standard_normal(50).astype(np.float32)
    pos = rng.permutation(50)
    assert list(O.select_keep(sc, pos, 50, 30, 2, 5, 0.0)) == \
        list(O.select_keep(sc, pos, 50, 30, 2, 5))
    # equal scores: decay evicts the oldest eligible positions first
    flat = np.ones(50, np.float32)
    keep = O.select_keep(flat, np.arange(50), 50, 30, 2, 5, -1e-3)
    assert list(keep) == [0, 1] + list(range(22, 50))


def test_decay_incremental_loop_equals_closed_form():
    rng = np.random.default_rng(33)
    for (B, S, W, L, n0) in ((20, 2, 4, 1, 30), (20, 2, 4, 5, 30),
                             (32, 4, 8, 8, 31)):
        lg = float(np.log(0.9))
        pol = O.Policy(B, S, W, L, log_gamma=(lg,))
        steps = 60
        sc = rng.standard_normal(n0 + steps).astype(np.float32)
        for newest, pe, kept in run_incremental(pol, n0, steps, sc):
            cf = O.closed_form_retained(sc[:newest + 1], newest, pe, pol, lg)
            np.testing.assert_array_equal(kept, cf)


# ---------------------------------------------------------------------------
# Stateful mLSTM scorer (KVpop section 3.3, Appendix A, E.3-E.4)
# ---------------------------------------------------------------------------

def _mlstm_weights(rng, d, P, bias_f=0.5, scale=1.0):
    r = lambda *s: rng.standard_normal(s) / np.sqrt(2 * d) * scale
    return O.MlstmWeights(r(P, 2 * d), r(P, 2 * d), r(P, 2 * d), r(2 * d),
                          r(2 * d), 0.1, bias_f, rng.standard_normal(P), 0.2)


def _recurrent_scores(weights, x, window):
    sc = O.MlstmScorer(weights, window)
    out = {}
    for t in range(x.shape[0]):
        r = sc.push(x[t])
        if r is not None:
            out[r[0]] = r[1]
    return out


def check_mlstm_hand(scorer_cls):
    g = golden()["mlstm_scalar"]
    z2 = np.zeros((1, 2))
    w = O.MlstmWeights(z2, z2, np.array([[1.0, 0.0]]), np.zeros(2),
                       np.zeros(2), 0.0, 0.0, np.array([1.0]), 0.0)
    sc = scorer_cls(w, g["window"])
    got = None
    for v in g["v"]:
        r = sc.push(np.array([v, 0.0]))
        if r is not None and r[0] == 0:
            got = r[1]
    assert got == pytest.approx(g["expected_u0"], rel=1e-12)


def check_mlstm_recurrent_equals_parallel(scorer_cls):
    rng = np.random.default_rng(41)
    for d, P, W, n in ((8, 4, 3, 30), (16, 8, 5, 40), (4, 2, 0, 12)):
        w = _mlstm_weights(rng, d, P)
        x = rng.standard_normal((n, 2 * d))
        sc = scorer_cls(w, W)
        rec = {}
        for t in range(n):
            r = sc.push(x[t])
            if r is not None:
                rec[r[0]] = r[1]
        par = O.mlstm_scores_parallel(x, w, W)
        assert sorted(rec) == list(range(n - W))
        np.testing.assert_allclose([rec[u] for u in range(n - W)], par,
                                   rtol=1e-11, atol=1e-12)


def test_mlstm_hand_case():
    check_mlstm_hand(O.MlstmScorer)


def test_mlstm_recurrent_equals_parallel_form():
    check_mlstm_recurrent_equals_parallel(O.MlstmScorer)


def test_mlstm_unit_gates_reduce_to_linear_attention():
    """i = f = 1 (zero gate weights, forget bias -> large) turns the state
    into linear attention with Hedgehog features (KVpop Appendix A): the
    readout is the similarity-weighted mean of the values."""
    rng = np.random.default_rng(42)
    d, P, W, n = 8, 4, 4, 25
    w = _mlstm_weights(rng, d, P)
    w.wi[:] = 0.0
    w.wf[:] = 0.0
    w.bi = 0.0
    w.bf = 60.0   # sigmoid(60) == 1 in float64
    x = rng.standard_normal((n, 2 * d))
    rec = _recurrent_scores(w, x, W)
    qf = O.hedgehog(x @ w.wq.T)
    kf = O.hedgehog(x @ w.wk.T)
    vf = x @ w.wv.T
    for u in range(n - W):
        q = u + W
        sim = kf[:q + 1] @ qf[u]
        h = (sim @ vf[:q + 1]) / sim.sum()
        ref = float(w.a @ (h * scipy.special.expit(h)) + w.b)
        assert rec[u] == pytest.approx(ref, rel=1e-12)


def test_hedgehog_feature_map():
    rng = np.random.default_rng(43)
    y = rng.standard_normal((5, 6))
    f = O.hedgehog(y)
    np.testing.assert_allclose(f[:, :6].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(f[:, 6:].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(f[:, :6], scipy.special.softmax(y, axis=1),
                               rtol=1e-14)
    np.testing.assert_allclose(O.hedgehog(-y), np.concatenate(
        [f[:, 6:], f[:, :6]], axis=1), rtol=1e-14)


# ---------------------------------------------------------------------------
# Prefill selection: ranks, running top-k cutoff, Eq. (26) mask, attention
# ---------------------------------------------------------------------------

def check_prefill_hand(ranks_fn, cutoffs_fn, mask_fn):
    g = golden()["prefill_cutoff"]
    s = np.asarray(g["scores"], np.float32)
    r = ranks_fn(s)
    assert r.tolist() == g["expected_rank"]
    tau = cutoffs_fn(r, g["sinks"], g["window"], g["k"])
    assert tau.tolist() == g["expected_tau"]
    M = mask_fn(r, tau, g["sinks"], g["window"])
    assert np.flatnonzero(M[7]).tolist() == g["expected_row7"]
    assert np.flatnonzero(M[4]).tolist() == g["expected_row4"]


def brute_force_ranks(s32, log_gamma=None):
    n = s32.shape[0]
    key = O.static_priority(s32, np.arange(n), log_gamma).astype(np.float64)
    r = np.zeros(n, dtype=np.int64)
    for t in range(n):
        for u in range(n):
            if key[u] > key[t] or (key[u] == key[t] and u > t):
                r[t] += 1
    return r


def decode_loop_rows(s32, sinks, window, k, log_gamma=None):
    """Retained positions after each append of the L = 1 decode loop
    (OracleLayer), starting from the first token."""
    n = s32.shape[0]
    B = sinks + window + k
    lay = O.OracleLayer(np.zeros((1, 1, 1, 1)), np.zeros((1, 1, 1, 1)),
                        s32[None, None, :1],
                        O.Policy(B, sinks, window, 1,
                                 log_gamma=None if log_gamma is None
                                 else (log_gamma,)), 1)
    rows = [sorted(lay.pos[0, 0].tolist())]
    for q in range(1, n):
        lay.append(np.zeros((1, 1, 1)), np.zeros((1, 1, 1)),
                   s32[None, None, q])
        lay.maybe_evict()
        rows.append(sorted(lay.pos[0, 0].tolist()))
    return rows


def check_prefill_mask_equals_decode_loop(ranks_fn, cutoffs_fn, mask_fn):
    rng = np.random.default_rng(51)
    for (n, S, W, k, lg, alphabet) in ((40, 2, 5, 6, None, 4),
                                       (60, 0, 3, 10, None, 0),
                                       (50, 4, 0, 7, -0.01, 3),
                                       (30, 3, 4, 0, None, 0),
                                       (45, 1, 1, 1, -0.2, 5)):
        s = (rng.integers(0, alphabet, n) if alphabet
             else rng.standard_normal(n)).astype(np.float32)
        r = ranks_fn(s, lg)
        tau = cutoffs_fn(r, S, W, k)
        M = mask_fn(r, tau, S, W)
        rows = decode_loop_rows(s, S, W, k, lg)
        for q in range(n):
            assert np.flatnonzero(M[q]).tolist() == rows[q], (n, S, W, k, q)


def test_prefill_hand_case():
    check_prefill_hand(O.prefill_ranks, O.prefill_cutoffs, O.prefill_mask)


def test_prefill_ranks_brute_force():
    rng = np.random.default_rng(52)
    for lg in (None, -0.05):
        for alphabet in (2, 3, 0):
            n = 30
            s = (rng.integers(0, alphabet, n) if alphabet
                 else rng.standard_normal(n)).astype(np.float32)
            s[::7] = -0.0 if alphabet else s[::7]
            assert O.prefill_ranks(s, lg).tolist() == \
                brute_force_ranks(s, lg).tolist()


def test_prefill_mask_equals_l1_decode_loop():
    """Eq. (26) rows are the retained sets of the L = 1 decode loop: with
    static priorities the running top-k of E(q) is what per-token eviction
    keeps (KVpop section 3.2)."""
    check_prefill_mask_equals_decode_loop(O.prefill_ranks, O.prefill_cutoffs,
                                          O.prefill_mask)


def test_prefill_cutoff_monotone_and_budget():
    rng = np.random.default_rng(53)
    n, S, W, k = 200, 4, 16, 24
    r = O.prefill_ranks(rng.standard_normal(n).astype(np.float32))
    tau = O.prefill_cutoffs(r, S, W, k)
    defined = tau < n
    first = int(np.argmax(defined))
    assert defined[first:].all()
    assert np.all(np.diff(tau[first:]) <= 0)  # more eligible tokens: cutoff only tightens
    M = O.prefill_mask(r, tau, S, W)
    assert np.all(M.sum(axis=1) == np.minimum(np.arange(n) + 1, S + W + k))


def test_prefill_attention_dense_limit():
    """k >= n keeps every causal pair: the masked attention is causal
    attention (float64 scaled_dot_product_attention)."""
    import torch
    rng = np.random.default_rng(54)
    H, G, n, d = 2, 3, 33, 16
    Q = rng.standard_normal((H * G, n, d))
    K = rng.standard_normal((H, n, d))
    V = rng.standard_normal((H, n, d))
    r = O.prefill_ranks(rng.standard_normal(n).astype(np.float32))
    tau = O.prefill_cutoffs(r, 2, 3, n)
    M = np.stack([O.prefill_mask(r, tau, 2, 3)] * H)
    assert M[0].sum() == n * (n + 1) // 2
    out, lse = O.prefill_attention(Q, K, V, M, G)
    Kx = torch.from_numpy(np.repeat(K, G, axis=0))
    Vx = torch.from_numpy(np.repeat(V, G, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), Kx, Vx, is_causal=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    z = np.einsum("jqd,jtd->jqt", Q, Kx.numpy()) / np.sqrt(d)
    z = np.where(np.tril(np.ones((n, n), bool)), z, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=2),
                               rtol=1e-12)


def test_prefill_attention_rows_are_decode_attention():
    """Row q of the masked attention equals decode attention over the
    tokens the mask keeps at q."""
    rng = np.random.default_rng(55)
    H, G, n, d, S, W, k = 2, 2, 48, 8, 2, 5, 7
    Q = rng.standard_normal((H * G, n, d))
    K = rng.standard_normal((H, n, d))
    V = rng.standard_normal((H, n, d))
    r = O.prefill_ranks(rng.standard_normal(n).astype(np.float32))
    tau = O.prefill_cutoffs(r, S, W, k)
    M1 = O.prefill_mask(r, tau, S, W)
    out, lse = O.prefill_attention(Q, K, V, np.stack([M1] * H), G)
    for q in (0, 9, 20, 47):
        keep = np.flatnonzero(M1[q])
        for j in range(H * G):
            o, l = O.decode_attention(Q[j, q][None], K[j // G, keep],
                                      V[j // G, keep])
            np.testing.assert_allclose(out[j, q], o[0], rtol=1e-12, atol=1e-14)
            assert lse[j, q] == pytest.approx(float(l[0]), rel=1e-12)


# ---------------------------------------------------------------------------
# Sink-attention gate (Fast KVzip section 3.4)
# ---------------------------------------------------------------------------

def _sink_weights(rng, D, H, G, dp, S, b=None):
    return O.SinkGateWeights(rng.standard_normal((H, dp, D)) / np.sqrt(D),
                             rng.standard_normal((H, G, dp, D)) / np.sqrt(D),
                             0.5 + rng.random(dp), 0.5 + rng.random(dp),
                             rng.standard_normal((S, dp)),
                             rng.random((H, G)) if b is None else b)


def _torch_qk(x, w):
    """q [n][H][G][D'], k [n][H][D'] by torch float64 linear + rms_norm."""
    import torch
    X = torch.from_numpy(np.asarray(x, np.float64))
    Wk = torch.from_numpy(np.asarray(w.wk, np.float64))
    Wq = torch.from_numpy(np.asarray(w.wq, np.float64))
    H, G, dp, D = Wq.shape
    k = torch.nn.functional.rms_norm(
        (X @ Wk.reshape(H * dp, D).T).reshape(-1, H, dp), (dp,),
        torch.from_numpy(np.asarray(w.gk, np.float64)), w.eps)
    q = torch.nn.functional.rms_norm(
        (X @ Wq.reshape(H * G * dp, D).T).reshape(-1, H, G, dp), (dp,),
        torch.from_numpy(np.asarray(w.gq, np.float64)), w.eps)
    return q.numpy(), k.numpy()


def check_sink_gate_hand(score_fn):
    g = golden()["sink_gate"]
    w = O.SinkGateWeights(np.eye(2)[None], np.eye(2)[None, None], np.ones(2),
                          np.ones(2), np.asarray([g["sink"]]),
                          np.full((1, 1), g["b"]), eps=0.0)
    got = score_fn(np.asarray([g["hidden"]]), w)
    assert got.shape == (1, 1)
    assert got[0, 0] == pytest.approx(g["expected"], rel=1e-12)


def check_sink_gate_without_denominator_is_sigmoid(score_fn):
    """No sink keys and b = 1 (the variant with sum_r exp(c_jr) + b_j = 1):
    each query head gives sigmoid(q_j . k_h / sqrt(D')); the KV head takes
    the largest."""
    rng = np.random.default_rng(61)
    D, H, G, dp = 24, 3, 2, 4
    w = _sink_weights(rng, D, H, G, dp, 0, b=np.ones((H, G)))
    x = rng.standard_normal((7, D))
    q, k = _torch_qk(x, w)
    a = np.einsum("nhgp,nhp->nhg", q, k) / np.sqrt(dp)
    np.testing.assert_allclose(score_fn(x, w),
                               scipy.special.expit(a).max(axis=-1),
                               rtol=1e-12)


def check_sink_gate_sinks_equal_to_key(score_fn):
    """Sink keys all equal to the token's own key and b = 0: the token's
    term competes with S identical terms, so every gate is 1 / (1 + S)."""
    rng = np.random.default_rng(62)
    D, dp, S = 16, 4, 5
    w = _sink_weights(rng, D, 1, 3, dp, S, b=np.zeros((1, 3)))
    x = rng.standard_normal((1, D))
    _, k = _torch_qk(x, w)
    w.sinks = np.repeat(k[0], S, axis=0)
    assert score_fn(x, w)[0, 0] == pytest.approx(1.0 / (1 + S), rel=1e-12)


def test_rms_norm_matches_torch():
    import torch
    rng = np.random.default_rng(60)
    y = rng.standard_normal((5, 3, 8))
    wt = rng.random(8)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y), (8,),
                                       torch.from_numpy(wt), 1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(y, wt, 1e-6), ref, rtol=1e-13)


def test_sink_gate_hand_case():
    check_sink_gate_hand(O.sink_gate_score)


def test_sink_gate_without_denominator_is_sigmoid():
    check_sink_gate_without_denominator_is_sigmoid(O.sink_gate_score)


def test_sink_gate_sinks_equal_to_key():
    check_sink_gate_sinks_equal_to_key(O.sink_gate_score)


def test_sink_gate_range_and_monotone_in_b():
    rng = np.random.default_rng(63)
    w = _sink_weights(rng, 32, 2, 4, 16, 16)
    x = rng.standard_normal((20, 32))
    g1 = O.sink_gate_score(x, w)
    assert np.all((g1 > 0) & (g1 < 1))
    w.b = w.b + 1.0
    assert np.all(O.sink_gate_score(x, w) < g1)


# ---------------------------------------------------------------------------
# Stochastic eviction (ForesightKV's Top-K multinomial rule)
# ---------------------------------------------------------------------------

def check_stochastic_zero_noise_is_greedy(fn):
    """Zero noise evicts the r lowest keys of the pool, which are the r
    lowest of all candidates: the deterministic rule (itself pinned by brute
    force above), over 3-valued scores with ties at the cut and decay."""
    rng = np.random.default_rng(71)
    for trial in range(300):
        n = int(rng.integers(4, 24))
        sc = rng.integers(0, 3, n).astype(np.float32)
        pos = rng.permutation(n + 5)[:n]
        S, W = int(rng.integers(0, 3)), int(rng.integers(0, 4))
        lg = None if trial % 3 else -0.25
        n_cand = int(O.eligible_mask(pos, S, W).sum())
        if n_cand == 0:
            continue
        n_keep = n - int(rng.integers(1, n_cand + 1))
        got = fn(sc, pos, n, n_keep, S, W, np.zeros(n, np.float32),
                 log_gamma=lg)
        ref = O.select_keep(sc, pos, n, n_keep, S, W, log_gamma=lg)
        np.testing.assert_array_equal(got, ref)


def check_stochastic_pool(fn):
    """Whatever the noise: exactly r candidates are evicted, all from the 2r
    lowest (brute-force count of candidates ranked below each), and the
    sinks and the window stay."""
    rng = np.random.default_rng(72)
    for _ in range(300):
        n = int(rng.integers(6, 30))
        sc = rng.integers(0, 4, n).astype(np.float32)
        pos = rng.permutation(n)
        S, W = 2, 3
        cand = np.nonzero(O.eligible_mask(pos, S, W))[0]
        r = int(rng.integers(1, cand.size + 1))
        g = (rng.standard_normal(n) * 50).astype(np.float32)
        keep = fn(sc, pos, n, n - r, S, W, g)
        evicted = np.setdiff1d(np.arange(n), keep)
        assert evicted.size == r and np.all(np.isin(evicted, cand))
        for e in evicted:
            below = sum(1 for c in cand if (sc[c], pos[c]) < (sc[e], pos[e]))
            assert below < 2 * r


def check_stochastic_distribution(fn):
    """The draw follows successive sampling without replacement with
    probability proportional to exp(-score) over the pool: frequencies of
    each evicted pair over 20000 numpy Gumbel draws against the exact
    two-draw probabilities p_a p_b (1/(1 - p_a) + 1/(1 - p_b))."""
    sc = np.array([9.0, 0.3, -0.5, 1.2, 0.0, 2.0, 9.0], np.float32)
    pos = np.arange(7)
    pool = [1, 2, 3, 4]        # the 4 lowest of candidates 1..5 (S = W = 1)
    w = np.exp(-sc[pool].astype(np.float64))
    p = dict(zip(pool, w / w.sum()))
    rng = np.random.default_rng(73)
    N = 20000
    counts = {}
    for _ in range(N):
        keep = fn(sc, pos, 7, 5, 1, 1, rng.gumbel(size=7).astype(np.float32))
        ev = tuple(np.setdiff1d(pos, keep))
        counts[ev] = counts.get(ev, 0) + 1
    assert set(counts) <= set(itertools.combinations(pool, 2))
    for a, b in itertools.combinations(pool, 2):
        exact = p[a] * p[b] * (1 / (1 - p[a]) + 1 / (1 - p[b]))
        sigma = math.sqrt(exact * (1 - exact) / N)
        assert abs(counts.get((a, b), 0) / N - exact) < 5 * sigma + 1e-4


def check_stochastic_hand(fn):
    """Hand case: scores [5, 1, 2, 0, 3, 4] at positions 0..5, S = 1, W = 1,
    keep 4 (r = 2). Candidates 1..4, pool = the 4 lowest = {3 (0), 1 (1),
    2 (2), 4 (3)}. Noise [0, 0.5, 3.5, 0.25, 1.0, 0]: sums -key + g = 1: -0.5,
    2: 1.5, 3: 0.25, 4: -2.0. The two largest, slots 2 and 3, are evicted."""
    keep = fn(np.array([5, 1, 2, 0, 3, 4], np.float32), np.arange(6), 6, 4, 1,
              1, np.array([0, 0.5, 3.5, 0.25, 1.0, 0], np.float32))
    np.testing.assert_array_equal(keep, [0, 1, 4, 5])


def test_stochastic_zero_noise_is_greedy():
    check_stochastic_zero_noise_is_greedy(O.select_keep_stochastic)


def test_stochastic_pool():
    check_stochastic_pool(O.select_keep_stochastic)


def test_stochastic_distribution():
    check_stochastic_distribution(O.select_keep_stochastic)


def test_stochastic_hand_case():
    check_stochastic_hand(O.select_keep_stochastic)
