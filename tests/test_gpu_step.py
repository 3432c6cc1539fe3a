"""a6 fused decode step end to end (kve_step through the C ABI) against the
float64 oracle's incremental policy loop, on inputs drawn on the host from
the synthetic module.

Every step checks: retained positions of every slice equal the oracle's
(except tokens whose oracle score lies within 1e-3 of the cut), GPU scores
within 1e-3 of the oracle's, and attention outputs within 2e-3 * max|out|
(computed by the oracle over the GPU's retained set when a tie made the sets
differ; the oracle is then resynchronised to that set).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import (attn_close, kve, oracle_gate_scores, oracle_mlp_scores,
                       shape_of, SCORE_ATOL, Tracker)

pytestmark = pytest.mark.gpu


def run_e2e(w, seed=0, check_stride=1, layer=0, gammas=None):
    import torch
    k = kve()
    dev = torch.device("cuda")
    mlp = w.scorer == "mlp"
    ctx = syn.initial_context(w, seed, layer)
    if mlp:
        wts = syn.draw_mlp_weights(w, seed, layer, biases=True)
        s0 = oracle_mlp_scores(ctx["k0"].f64, ctx["v0"].f64, wts, w.act)
        sc = k.Scorer.mlp(wts["w1"].torch(dev), wts["w2"].torch(dev),
                          wts["b1"].torch(dev), wts["b2"].torch(dev),
                          act=k.ACT_RELU if w.act == "relu" else k.ACT_SILU)
    else:
        gw = syn.draw_gate_weights(w, seed, layer, bias=True)
        s0 = oracle_gate_scores(ctx["hidden0"].f64, gw)
        sc = k.Scorer.gate(gw["w"].torch(dev), gw["b"].torch(dev))
    lg = None
    if gammas is not None:
        lg = np.log(np.asarray(gammas, np.float64)).astype(np.float32)
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len,
                     log_gamma=None if lg is None else tuple(float(x) for x in lg))
    tr = Tracker(w, ctx["k0"].f64, ctx["v0"].f64, s0, pol_o)

    shape = shape_of(w)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len,
                   log_gamma=None if lg is None else torch.from_numpy(lg).to(dev))
    cache = k.CacheTensors.empty(shape, dev)
    cache.k[:, :, :w.n0] = ctx["k0"].torch(dev)
    cache.v[:, :, :w.n0] = ctx["v0"].torch(dev)
    cache.pos[:, :, :w.n0] = torch.arange(w.n0, dtype=torch.int32, device=dev)
    keep = torch.zeros((w.batch, w.n_kv, w.capacity), dtype=torch.int32,
                       device=dev)
    ws = k.alloc_workspace(shape, w.capacity, dev)
    hbuf = None
    if mlp:
        k.kve_score(shape, sc, cache, 0, w.n0)
    else:
        k.kve_score(shape, sc, cache, 0, w.n0, hidden=ctx["hidden0"].torch(dev))
        hbuf = torch.zeros((w.batch, w.evict_len, w.hidden),
                           dtype=torch.bfloat16, device=dev)
    got_s = cache.score[:, :, :w.n0].cpu().numpy()
    np.testing.assert_allclose(got_s, s0, rtol=0, atol=SCORE_ATOL)
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
    G = w.group
    evictions = 0
    for i in range(w.steps):
        st = syn.step_inputs(w, seed, layer, i)
        if mlp:
            sn = oracle_mlp_scores(st["k_new"].f64[:, :, None],
                                   st["v_new"].f64[:, :, None], wts,
                                   w.act)[:, :, 0]
            k.kve_step(shape, pol, sc, cache, state, st["k_new"].torch(dev),
                       st["v_new"].torch(dev), st["q"].torch(dev), out, lse,
                       keep, ws)
        else:
            sn = oracle_gate_scores(st["hidden_new"].f64[:, None], gw)[:, :, 0]
            k.kve_step(shape, pol, sc, cache, state, st["k_new"].torch(dev),
                       st["v_new"].torch(dev), st["q"].torch(dev), out, lse,
                       keep, ws, hidden_new=st["hidden_new"].torch(dev),
                       hidden_buf=hbuf)
        tr.step(w.n0 + i, st["k_new"].f64, st["v_new"].f64, sn)
        evictions += state.evicted
        if i % check_stride and not state.evicted and i != w.steps - 1:
            continue
        torch.cuda.synchronize()
        gpu_pos = cache.pos[:, :, :state.len].cpu().numpy().astype(np.int64)
        assert state.len == tr.lay.n
        tr.check_and_sync(gpu_pos)
        if state.evicted:
            # scores of the retained entries match the oracle's by position
            gs = cache.score[:, :, :state.len].cpu().numpy()
            ref = np.take_along_axis(tr.S, gpu_pos, axis=2)
            np.testing.assert_allclose(gs, ref, rtol=0, atol=SCORE_ATOL)
        ref_out, _ = tr.lay.attend(st["q"].f64)
        attn_close(out.cpu().double().numpy(), ref_out, f"step {i}")
    return evictions, tr


def test_tiny_workload_full_run():
    """Config 1: fp32, d=64, G=2, n0=512 -> B=192, L=1, 64 steps."""
    w = syn.workload(1)
    print(f"[step] {w.name}", flush=True)
    ev, _ = run_e2e(w)
    assert ev == w.steps  # L = 1 evicts at every step once saturated


def test_tiny_workload_other_seed():
    w = syn.workload(1, steps=16)
    run_e2e(w, seed=1)


@pytest.mark.parametrize("seed", [0, 1])
def test_qwen3_layer_structured(seed):
    """Config 2 shapes (structured rows, heavy hitters), batch cut to 2:
    n0=8192 -> B=1024, L=128, 256 steps (two periodic evictions)."""
    w = syn.workload(2, batch=2)
    print(f"[step] {w.name} batch=2 seed={seed}", flush=True)
    ev, _ = run_e2e(w, seed=seed, check_stride=8)
    assert ev == 2


def test_qwen3_layer_full_batch():
    """Config 2 as specified: batch 16 (128 slices, split attention), the
    structured rows with heavy hitters, n0 = 8192 -> B = 1024, L = 128, 256
    steps with the evictions at steps 128 and 256; every slice checked on
    every 16th step and on each evicting step."""
    w = syn.workload(2)
    assert w.batch == 16
    print(f"[step] {w.name} batch={w.batch}", flush=True)
    ev, _ = run_e2e(w, seed=2, check_stride=16)
    assert ev == 2


def test_qwen3_layer_silu_and_odd_policy():
    w = syn.workload(2, batch=1, n0=700, budget=300, sinks=3, window=37,
                     evict_len=45, steps=100, act="silu", structured=False)
    ev, _ = run_e2e(w, seed=3)
    assert ev == 2


def test_temporal_decay_end_to_end():
    """KVpop temporal decay (decay step 1, per-head gamma in the Table 3
    range and below it) through kve_step, tiny and Qwen3-4B-layer shapes."""
    w = syn.workload(1, steps=48)
    ev, _ = run_e2e(w, seed=5, gammas=[0.99, 0.999999])
    assert ev == w.steps
    w = syn.workload(2, batch=1, steps=256)
    ev, _ = run_e2e(w, seed=6, check_stride=8,
                    gammas=np.linspace(0.999, 0.999999, 8))
    assert ev == 2


def test_no_eviction_equals_dense_attention():
    """B above the context: nothing is evicted, the step is dense decode."""
    w = syn.workload(2, batch=1, n0=200, budget=600, window=64, evict_len=64,
                     steps=40, structured=False)
    ev, tr = run_e2e(w, seed=4)
    assert ev == 0
    assert tr.lay.n == 240


def test_gate_scorer_workload():
    """Config 5 structure (gate on 5120-dim hidden states, G=5, W=512,
    L=64) at a reduced prompt: n0=4096 -> 30% budget, 130 steps."""
    w = syn.workload(5, n0=4096, budget=int(0.3 * 4096), steps=130)
    print(f"[step] gate n0=4096 B={w.budget}", flush=True)
    ev, _ = run_e2e(w, seed=0, check_stride=4)
    assert ev == 2


def test_checkpoint_resume_bitwise():
    """Save the device state mid-run, continue, restore, replay: identical
    outputs and caches (the decode state is K, V, score, pos and len)."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(2, batch=1, n0=1500, steps=300, structured=False)
    ctx = syn.initial_context(w, 0, 0)
    wts = syn.draw_mlp_weights(w, 0, 0)
    shape = shape_of(w)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    sc = k.Scorer.mlp(wts["w1"].torch(dev), wts["w2"].torch(dev))
    cache = k.CacheTensors.empty(shape, dev)
    cache.k[:, :, :w.n0] = ctx["k0"].torch(dev)
    cache.v[:, :, :w.n0] = ctx["v0"].torch(dev)
    cache.pos[:, :, :w.n0] = torch.arange(w.n0, dtype=torch.int32, device=dev)
    keep = torch.zeros((1, w.n_kv, w.capacity), dtype=torch.int32, device=dev)
    ws = k.alloc_workspace(shape, w.capacity, dev)
    k.kve_score(shape, sc, cache, 0, w.n0)
    k.kve_select_evict(shape, pol, cache, w.n0, w.budget, keep)
    k.kve_compact(shape, cache, w.n0, keep, w.budget)
    state = k.DecodeState(w.budget, w.budget, w.n0)
    out = torch.zeros((1, w.n_q, w.head_dim), device=dev)
    inputs = [syn.step_inputs(w, 0, 0, i) for i in range(w.steps)]

    def run(i0, i1, st):
        outs = []
        for i in range(i0, i1):
            x = inputs[i]
            k.kve_step(shape, pol, sc, cache, st, x["k_new"].torch(dev),
                       x["v_new"].torch(dev), x["q"].torch(dev), out, None,
                       keep, ws)
            outs.append(out.clone())
        return outs

    first = run(0, 100, state)
    snap = (cache.k.clone(), cache.v.clone(), cache.score.clone(),
            cache.pos.clone(), k.DecodeState(**vars(state)))
    a = run(100, w.steps, state)
    cache.k.copy_(snap[0]); cache.v.copy_(snap[1])
    cache.score.copy_(snap[2]); cache.pos.copy_(snap[3])
    b = run(100, w.steps, snap[4])
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert first  # the first leg ran


def _graph_case(k, dev, evicting):
    """A batch-8 layer (64 slices, split attention) one step short of an
    eviction, or ten steps past one."""
    import torch
    batch, H, G, D, B, L, S, W = 8, 8, 4, 128, 512, 64, 4, 64
    gen = torch.Generator().manual_seed(17 + evicting)
    cap = B + L
    shape = k.Shape(batch, H, G, D, cap, k.BF16)
    pol = k.Policy(B, S, W, L)
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(torch.randn(cache.k.shape, generator=gen).to(torch.bfloat16))
    cache.v.copy_(torch.randn(cache.v.shape, generator=gen).to(torch.bfloat16))
    cache.score.copy_(torch.randn(cache.score.shape, generator=gen))
    cache.pos.copy_(torch.arange(cap, dtype=torch.int32).expand(batch, H, cap))
    w1 = (torch.randn((H, 64, 2 * D), generator=gen) * (2 * D) ** -0.5
          ).to(torch.bfloat16).to(dev)
    w2 = (torch.randn((H, 64), generator=gen) * 64 ** -0.5).to(dev)
    sc = k.Scorer.mlp(w1, w2)
    n = B + L - 1 if evicting else B + 10
    x = [torch.randn(s_, generator=gen).to(torch.bfloat16).to(dev)
         for s_ in ((batch, H, D), (batch, H, D), (batch, H * G, D))]
    return shape, pol, sc, cache, n, x


@pytest.mark.parametrize("evicting", [False, True], ids=["append", "evict"])
def test_step_in_hip_graph(evicting):
    """kve_step's launches replay from a captured HIP graph: the fused append
    and split attention of a plain step, or the append, scoring, select,
    compaction and attention of an evicting one. The library allocates
    nothing and records no memset. Each replay runs on the cache restored
    from its pre-step snapshot (eager copies and synchronisations between
    replays) and must leave the cache, the kept slots and the outputs
    bitwise equal to the eager step's."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    print(f"[step-graph] evicting={evicting}", flush=True)
    shape, pol, sc, cache, n, (kn, vn, q) = _graph_case(k, dev, evicting)
    B = pol.budget
    ws = k.alloc_workspace(shape, shape.capacity, dev)
    snap = [t.clone() for t in (cache.k, cache.v, cache.score, cache.pos)]

    def restore():
        for t, s_ in zip((cache.k, cache.v, cache.score, cache.pos), snap):
            t.copy_(s_)

    out = torch.empty((shape.batch, shape.n_kv_heads * shape.group,
                       shape.head_dim), device=dev)
    lse = torch.empty(out.shape[:2], device=dev)
    keep = torch.full((shape.batch, shape.n_kv_heads, B), -1,
                      dtype=torch.int32, device=dev)
    st = k.DecodeState(n, B, n)
    k.kve_step(shape, pol, sc, cache, st, kn, vn, q, out, lse, keep, ws)
    torch.cuda.synchronize()
    assert st.evicted == int(evicting)
    want = [t.clone() for t in (cache.k, cache.v, cache.score, cache.pos,
                                out, lse, keep)]

    restore()
    torch.cuda.synchronize()
    g_state = k.DecodeState(n, B, n)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            k.kve_step(shape, pol, sc, cache, g_state, kn, vn, q, out, lse,
                       keep, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert (g_state.len, g_state.evicted) == (st.len, st.evicted)
    other = torch.empty_like(out)
    for rep in range(3):
        restore()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        keep.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (cache.k, cache.v, cache.score, cache.pos, out, lse, keep)
        for name, a, b in zip(("k", "v", "score", "pos", "out", "lse", "keep"),
                              got, want):
            same = torch.equal(a.view(torch.int16), b.view(torch.int16)) \
                if a.dtype == torch.bfloat16 else torch.equal(a, b)
            assert same, f"replay {rep}: {name} differs"
        # eager work on the same workspace between replays
        k.kve_decode_attn(shape, cache, B, q, other, None, ws)
        torch.cuda.synchronize()
