"""Stateful mLSTM scorer with delayed read-out (KVpop section 3.3, Appendix
E.3-E.4) through the C ABI, against the oracle's plain float64 recurrence.

Scores are compared by token position within MLSTM_ATOL. The GPU keeps the
recurrent state in float32 with a lazily renormalised log scale; both sides
read the same bf16 inputs and weights, and the projections accumulate in
float32 on the GPU. The read-out h is a ratio of positive-weighted sums, so
its error is a few float32 roundings relative to max |v~| (about 5); with
|a|_1 about 6 the score error stays below 1e-4, and MLSTM_ATOL = 2e-4 leaves
a factor of two.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import (attn_close, kve, mlstm_device_scorer,
                       oracle_mlstm_weights, SCORE_ATOL, Tracker)

pytestmark = pytest.mark.gpu

MLSTM_ATOL = 2e-4
UNSET = 12345.0


def oracle_scores(K, V, wts, delay):
    """Scores by position of tokens 0..n-1 of every slice (NaN: not read
    out), K, V [b][H][n][d] float64 in position order."""
    b, H, n, _ = K.shape
    out = np.full((b, H, n), np.nan)
    for bi in range(b):
        for h in range(H):
            sc = O.MlstmScorer(oracle_mlstm_weights(wts, h), delay)
            for t in range(n):
                r = sc.push(np.concatenate([K[bi, h, t], V[bi, h, t]]))
                if r is not None:
                    out[bi, h, r[0]] = r[1]
    return out


def by_position(vals, pos, n):
    b, H, _ = vals.shape
    out = np.full((b, H, n), np.nan)
    for bi in range(b):
        for h in range(H):
            p = pos[bi, h]
            ok = (p >= 0) & (p < n)
            out[bi, h, p[ok]] = vals[bi, h][ok]
    return out


CASES = [
    # batch, H, d, n, W, absorb cuts (one kve_score call per range)
    (2, 3, 128, 300, 128, (300,)),
    (1, 2, 64, 200, 16, (200,)),
    (1, 2, 128, 77, 0, (77,)),           # W = 0: read out at absorption
    (1, 2, 128, 50, 64, (50,)),          # nothing leaves the window yet
    (2, 2, 128, 400, 64, (37, 200, 233, 400)),
    (1, 2, 64, 300, 100, (1, 2, 150, 151, 300)),
    (1, 1, 128, 129, 128, (128, 129)),   # one read-out, found by lookup
]


def run_case(b, H, d, n, W, cuts, seed, gate_b=None, wscale=None):
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(2, batch=b, n_kv=H, head_dim=d, scorer="mlstm",
                     hidden=d // 2)
    rng = np.random.default_rng(seed)
    K = syn.Stored(rng.standard_normal((b, H, n, d)).astype(np.float32), "bf16")
    V = syn.Stored(rng.standard_normal((b, H, n, d)).astype(np.float32), "bf16")
    wts = syn.draw_mlstm_weights(w, seed, 0)
    if gate_b is not None or wscale is not None:
        wt = wts["w"].f64.astype(np.float32)
        P = d // 2
        if wscale is not None:
            wt[:, 3 * P:] *= wscale
        wts["w"] = syn.Stored(wt, "bf16")
        if gate_b is not None:
            wts["gate_b"] = syn.Stored(np.broadcast_to(
                np.asarray(gate_b, np.float32), (H, 2)).copy(), "f32")
    shape = k.Shape(b, H, 1, d, n, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(K.torch(dev))
    cache.v.copy_(V.torch(dev))
    cache.pos.copy_(torch.arange(n, dtype=torch.int32, device=dev))
    cache.score.fill_(UNSET)
    sc = mlstm_device_scorer(wts, W, dev)
    cache.attach_scorer_state(shape, sc)
    prng = np.random.default_rng(seed + 1)
    prev = 0
    for cut in cuts:
        if prev > 1:
            # Older rows move between calls, as compaction moves them.
            perm = torch.from_numpy(prng.permutation(prev)).to(dev)
            for t in (cache.k, cache.v, cache.score, cache.pos):
                t[:, :, :prev] = t[:, :, perm]
        k.kve_score(shape, sc, cache, prev, cut)
        prev = cut
    torch.cuda.synchronize()
    ref = oracle_scores(K.f64, V.f64, wts, W)
    got = by_position(cache.score.cpu().numpy(),
                      cache.pos.cpu().numpy().astype(np.int64), n)
    read = ~np.isnan(ref)
    assert read.sum() == b * H * max(n - W, 0)
    err = float(np.max(np.abs(got[read] - ref[read]))) if read.any() else 0.0
    print(f"[mlstm] max |err| {err:.3g}", flush=True)
    np.testing.assert_allclose(got[read], ref[read], rtol=0, atol=MLSTM_ATOL)
    assert np.all(got[~read] == UNSET)
    return ref


@pytest.mark.parametrize("case", CASES, ids=[
    f"b{c[0]}H{c[1]}d{c[2]}n{c[3]}W{c[4]}calls{len(c[5])}" for c in CASES])
def test_mlstm_scores(case):
    print(f"[mlstm] {case}", flush=True)
    run_case(*case, seed=sum(case[:5]))


def test_mlstm_renormalises_under_steep_gates():
    """Input-gate preactivations spread over tens of units and a forget gate
    near 0.1: the log scale moves by about 2 per token, so the state is
    renormalised every few tokens."""
    print("[mlstm] steep gates", flush=True)
    run_case(1, 2, 128, 1000, 32, (400, 1000), seed=5, gate_b=(0.0, -2.0),
             wscale=8.0)


def test_mlstm_renormalises_between_chunks():
    """Forget gate near 1/2: the log scale falls by about 0.7 per token, so
    the chunk reference moves past the renormalisation threshold every few
    chunks while each chunk's spread stays small."""
    print("[mlstm] chunk renormalisation", flush=True)
    run_case(2, 2, 128, 1000, 64, (1000,), seed=7, gate_b=(0.0, 0.0))


def test_mlstm_long_memory():
    """Forget gate at 1 - 2e-9 (float32 rounds it to 1): a long sum without
    decay, 4096 tokens."""
    print("[mlstm] long memory", flush=True)
    run_case(1, 2, 128, 4096, 128, (4096,), seed=6, gate_b=(0.0, 20.0))


def run_e2e_mlstm(w, seed=0, check_stride=1, layer=0):
    """kve_step with the stateful scorer: retained sets, scores (at every
    eviction) and attention against the oracle's policy loop, the oracle
    scoring each token when it leaves the window."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    W = w.window
    ctx = syn.initial_context(w, seed, layer)
    wts = syn.draw_mlstm_weights(w, seed, layer)
    scorers = [[O.MlstmScorer(oracle_mlstm_weights(wts, h), W)
                for h in range(w.n_kv)] for _ in range(w.batch)]
    s0 = np.zeros((w.batch, w.n_kv, w.n0), np.float32)
    for bi in range(w.batch):
        for h in range(w.n_kv):
            for t in range(w.n0):
                r = scorers[bi][h].push(np.concatenate(
                    [ctx["k0"].f64[bi, h, t], ctx["v0"].f64[bi, h, t]]))
                if r is not None:
                    s0[bi, h, r[0]] = r[1]
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    tr = Tracker(w, ctx["k0"].f64, ctx["v0"].f64, s0, pol_o)

    shape = k.Shape(w.batch, w.n_kv, w.group, w.head_dim, w.capacity, k.BF16)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    sc = mlstm_device_scorer(wts, W, dev)
    cache = k.CacheTensors.empty(shape, dev)
    cache.attach_scorer_state(shape, sc)
    cache.k[:, :, :w.n0] = ctx["k0"].torch(dev)
    cache.v[:, :, :w.n0] = ctx["v0"].torch(dev)
    cache.pos[:, :, :w.n0] = torch.arange(w.n0, dtype=torch.int32, device=dev)
    keep = torch.zeros((w.batch, w.n_kv, w.capacity), dtype=torch.int32,
                       device=dev)
    ws = k.alloc_workspace(shape, w.capacity, dev)
    k.kve_score(shape, sc, cache, 0, w.n0)
    got_s = cache.score[:, :, :w.n0 - W].cpu().numpy()
    np.testing.assert_allclose(got_s, s0[:, :, :w.n0 - W], rtol=0,
                               atol=MLSTM_ATOL)
    tr.prefill()
    n = w.n0
    if w.n0 > w.budget:
        k.kve_select_evict(shape, pol, cache, w.n0, w.budget, keep)
        k.kve_compact(shape, cache, w.n0, keep, w.budget)
        n = w.budget
    tr.check_and_sync(cache.pos[:, :, :n].cpu().numpy().astype(np.int64))
    state = k.DecodeState(n, n, w.n0)
    out = torch.zeros((w.batch, w.n_q, w.head_dim), device=dev)
    lse = torch.zeros((w.batch, w.n_q), device=dev)
    evictions = 0
    for i in range(w.steps):
        st = syn.step_inputs(w, seed, layer, i)
        q_pos = w.n0 + i
        su = np.zeros((w.batch, w.n_kv), np.float32)
        for bi in range(w.batch):
            for h in range(w.n_kv):
                r = scorers[bi][h].push(np.concatenate(
                    [st["k_new"].f64[bi, h], st["v_new"].f64[bi, h]]))
                assert r is not None and r[0] == q_pos - W
                su[bi, h] = r[1]
        k.kve_step(shape, pol, sc, cache, state, st["k_new"].torch(dev),
                   st["v_new"].torch(dev), st["q"].torch(dev), out, lse,
                   keep, ws)
        tr.step(q_pos, st["k_new"].f64, st["v_new"].f64,
                np.zeros((w.batch, w.n_kv), np.float32),
                delayed=(q_pos - W, su))
        evictions += state.evicted
        if i % check_stride and not state.evicted and i != w.steps - 1:
            continue
        torch.cuda.synchronize()
        gpu_pos = cache.pos[:, :, :state.len].cpu().numpy().astype(np.int64)
        assert state.len == tr.lay.n
        tr.check_and_sync(gpu_pos)
        if state.evicted:
            # Every retained token that has left the window is scored.
            gs = cache.score[:, :, :state.len].cpu().numpy()
            ref = np.take_along_axis(tr.S, gpu_pos, axis=2)
            scored = gpu_pos <= q_pos - W
            np.testing.assert_allclose(gs[scored], ref[scored], rtol=0,
                                       atol=MLSTM_ATOL)
        ref_out, _ = tr.lay.attend(st["q"].f64)
        attn_close(out.cpu().double().numpy(), ref_out, f"step {i}")
    return evictions


def test_mlstm_step_evict_every_token():
    """Small bf16 layer (d = 64, G = 2) with L = 1: the stateful scorer
    absorbs one token per step and reads out the token leaving the window
    from wherever compaction put it."""
    w = syn.workload(1, kv_dtype="bf16", scorer="mlstm", hidden=32, steps=48)
    print(f"[mlstm-step] {w.name} bf16 L=1", flush=True)
    ev = run_e2e_mlstm(w)
    assert ev == w.steps


def test_mlstm_step_qwen3_layer():
    """Qwen3-4B layer shapes, batch 2: n0 = 8192 -> B = 1024, L = 128,
    W = 128, 256 steps (two periodic evictions, 128 tokens absorbed at
    each)."""
    w = syn.workload(2, batch=2, scorer="mlstm", hidden=64)
    print(f"[mlstm-step] {w.name} batch=2", flush=True)
    ev = run_e2e_mlstm(w, check_stride=16)
    assert ev == 2


def test_mlstm_full_size_prompt_and_flush_sampled():
    """The batch-96 Qwen3-4B layer in the benchmark's launch configuration:
    all 768 slices absorb an 8192-token prompt in one launch, then one
    buffered-scoring flush absorbs 128 more tokens and reads 128 out; six
    sampled slices (first, last and four others) against the oracle's
    float64 recurrence, every read-out score."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(4, scorer="mlstm", hidden=64)
    b, H, d, n0, L, W = w.batch, w.n_kv, w.head_dim, w.n0, w.evict_len, w.window
    n = n0 + L
    print(f"[mlstm-full] b={b} H={H} n0={n0} L={L}", flush=True)
    T = syn.TENSOR_IDS
    K = syn.device_normal((b, H, n, d), 4, (4, 0, 0, T["k0"]), torch.bfloat16, dev)
    V = syn.device_normal((b, H, n, d), 4, (4, 0, 0, T["v0"]), torch.bfloat16, dev)
    wts = syn.draw_mlstm_weights(w, 4, 0)
    shape = k.Shape(b, H, w.group, d, n, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(K)
    cache.v.copy_(V)
    cache.pos.copy_(torch.arange(n, dtype=torch.int32, device=dev).expand(b, H, n))
    cache.score.fill_(UNSET)
    sc = mlstm_device_scorer(wts, W, dev)
    cache.attach_scorer_state(shape, sc)
    k.kve_score(shape, sc, cache, 0, n0)       # prompt absorption
    k.kve_score(shape, sc, cache, n0, n)       # one flush of L tokens
    torch.cuda.synchronize()
    sampled = [(0, 0), (b - 1, H - 1), (17, 3), (40, 6), (63, 1), (90, 5)]
    for bi, h in sampled:
        Kh = K[bi, h].float().cpu().double().numpy()
        Vh = V[bi, h].float().cpu().double().numpy()
        scorer = O.MlstmScorer(oracle_mlstm_weights(wts, h), W)
        ref = np.full(n, np.nan)
        for t in range(n):
            r = scorer.push(np.concatenate([Kh[t], Vh[t]]))
            if r is not None:
                ref[r[0]] = r[1]
        got = cache.score[bi, h].cpu().numpy()
        read = ~np.isnan(ref)
        assert read.sum() == n - W
        err = float(np.max(np.abs(got[read] - ref[read])))
        print(f"[mlstm-full] slice ({bi},{h}) max |err| {err:.3g}", flush=True)
        np.testing.assert_allclose(got[read], ref[read], rtol=0, atol=MLSTM_ATOL)
        assert np.all(got[~read] == UNSET)
