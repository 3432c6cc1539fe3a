"""Low-rank sink-attention gate (Fast KVzip section 3.4) through the C ABI,
against the float64 oracle.

The projections run on MFMA with float32 accumulation of exact bf16
products, and the normalisation, sink softmax and gate in float32; the gate
lies in [0, 1] and its error is a few float32 roundings of the logits
(|logit| <~ 10), about 1e-6. SINK_GATE_ATOL = 2e-5 leaves a margin.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import (attn_close, kve, oracle_sink_gate_scores, SCORE_ATOL,
                       Tracker)

pytestmark = pytest.mark.gpu

SINK_GATE_ATOL = 2e-5

CASES = [
    # batch, H, G, D, rows, slot_begin, cap, n_sink
    (1, 8, 5, 5120, 300, 0, 300, 16),        # Qwen2.5-14B layer
    (1, 8, 5, 5120, 64, 39321, 39385, 16),   # a decode buffer of L = 64
    (2, 3, 2, 256, 77, 10, 100, 5),
    (1, 2, 1, 64, 130, 0, 130, 0),           # no sink keys
    (1, 4, 8, 1024, 200, 0, 200, 16),        # G = 8
    (1, 5, 3, 96, 517, 3, 600, 7),           # D % 64 == 32: a half k chunk
    (3, 7, 7, 160, 33, 0, 40, 16),           # G = 7, one partial block
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"b{c[0]}H{c[1]}G{c[2]}D{c[3]}r{c[4]}S{c[7]}" for c in CASES])
def test_sink_gate_scores(case):
    import torch
    k = kve()
    dev = torch.device("cuda")
    B, H, G, D, rows, s0, cap, S = case
    print(f"[sink-gate] {case}", flush=True)
    w = syn.workload(5, batch=B, n_kv=H, group=G, hidden=D, scorer="sink_gate")
    wts = syn.draw_sink_gate_weights(w, sum(case), 0, n_sink=S)
    rng = np.random.default_rng(sum(case))
    hid = syn.Stored(rng.standard_normal((B, rows, D)).astype(np.float32), "bf16")
    shape = k.Shape(B, H, G, 128, cap, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    cache.score.fill_(12345.0)
    sc = k.Scorer.sink_gate(wts["w"].torch(dev), wts["sinks"].torch(dev),
                            norm=wts["norm"].torch(dev), b=wts["b"].torch(dev))
    k.kve_score(shape, sc, cache, s0, s0 + rows, hidden=hid.torch(dev))
    got = cache.score.cpu().numpy()
    ref = oracle_sink_gate_scores(hid.f64, wts, H, G)
    err = float(np.abs(got[:, :, s0:s0 + rows] - ref).max())
    print(f"[sink-gate] max |err| {err:.3g}", flush=True)
    np.testing.assert_allclose(got[:, :, s0:s0 + rows], ref, rtol=0,
                               atol=SINK_GATE_ATOL)
    assert np.all(got[:, :, :s0] == 12345.0)
    assert np.all(got[:, :, s0 + rows:] == 12345.0)


def run_e2e_sink_gate(w, seed=0, layer=0, check_stride=16):
    """kve_step with the sink gate on hidden states (buffered scoring):
    retained sets, scores at every eviction and attention against the
    oracle's policy loop. Returns the number of evictions."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    ctx = syn.initial_context(w, seed, layer)
    wts = syn.draw_sink_gate_weights(w, seed, layer)
    s0 = oracle_sink_gate_scores(ctx["hidden0"].f64, wts, w.n_kv, w.group)
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    tr = Tracker(w, ctx["k0"].f64, ctx["v0"].f64, s0, pol_o)
    shape = k.Shape(w.batch, w.n_kv, w.group, w.head_dim, w.capacity, k.BF16)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    sc = k.Scorer.sink_gate(wts["w"].torch(dev), wts["sinks"].torch(dev),
                            norm=wts["norm"].torch(dev), b=wts["b"].torch(dev))
    cache = k.CacheTensors.empty(shape, dev)
    cache.k[:, :, :w.n0] = ctx["k0"].torch(dev)
    cache.v[:, :, :w.n0] = ctx["v0"].torch(dev)
    cache.pos[:, :, :w.n0] = torch.arange(w.n0, dtype=torch.int32, device=dev)
    k.kve_score(shape, sc, cache, 0, w.n0, hidden=ctx["hidden0"].torch(dev))
    np.testing.assert_allclose(cache.score[:, :, :w.n0].cpu().numpy(), s0,
                               rtol=0, atol=SINK_GATE_ATOL)
    keep = torch.zeros((w.batch, w.n_kv, w.capacity), dtype=torch.int32,
                       device=dev)
    ws = k.alloc_workspace(shape, w.capacity, dev)
    tr.prefill()
    n = w.n0
    if w.n0 > w.budget:
        k.kve_select_evict(shape, pol, cache, w.n0, w.budget, keep)
        k.kve_compact(shape, cache, w.n0, keep, w.budget)
        n = w.budget
    tr.check_and_sync(cache.pos[:, :, :n].cpu().numpy().astype(np.int64))
    state = k.DecodeState(n, n, w.n0)
    hbuf = torch.zeros((w.batch, w.evict_len, w.hidden), dtype=torch.bfloat16,
                       device=dev)
    out = torch.zeros((w.batch, w.n_q, w.head_dim), device=dev)
    lse = torch.zeros((w.batch, w.n_q), device=dev)
    evictions = 0
    for i in range(w.steps):
        st = syn.step_inputs(w, seed, layer, i)
        sn = oracle_sink_gate_scores(st["hidden_new"].f64[:, None], wts,
                                     w.n_kv, w.group)[:, :, 0]
        k.kve_step(shape, pol, sc, cache, state, st["k_new"].torch(dev),
                   st["v_new"].torch(dev), st["q"].torch(dev), out, lse, keep,
                   ws, hidden_new=st["hidden_new"].torch(dev), hidden_buf=hbuf)
        tr.step(w.n0 + i, st["k_new"].f64, st["v_new"].f64, sn)
        evictions += state.evicted
        if i % check_stride and not state.evicted and i != w.steps - 1:
            continue
        torch.cuda.synchronize()
        gpu_pos = cache.pos[:, :, :state.len].cpu().numpy().astype(np.int64)
        assert state.len == tr.lay.n
        tr.check_and_sync(gpu_pos)
        if state.evicted:
            gs = cache.score[:, :, :state.len].cpu().numpy()
            ref = np.take_along_axis(tr.S, gpu_pos, axis=2)
            np.testing.assert_allclose(gs, ref, rtol=0, atol=SINK_GATE_ATOL)
        ref_out, _ = tr.lay.attend(st["q"].f64)
        attn_close(out.cpu().double().numpy(), ref_out, f"step {i}")
    return evictions


def test_sink_gate_step_end_to_end():
    """kve_step with the sink gate on hidden states (buffered scoring): the
    Qwen2.5-14B layer shape cut to a 4096-token prompt, B = 1024, W = 128,
    L = 64, 200 steps."""
    w = syn.workload(5, n0=4096, budget=1024, window=128, steps=200,
                     scorer="sink_gate")
    print(f"[sink-gate-step] {w.name}", flush=True)
    assert run_e2e_sink_gate(w) == 3


def test_sink_gate_full_prompt_sampled():
    """The whole 131072-token Qwen2.5-14B prompt (D = 5120, 8 KV heads, 40
    query heads, S = 16) in one launch, as the gate benchmark times it; 600
    sampled tokens, the last 64 among them, against the oracle."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(5, scorer="sink_gate")
    H, G, D, n = w.n_kv, w.group, w.hidden, w.n0
    print(f"[sink-gate-full] n={n} D={D} H={H} G={G}", flush=True)
    T = syn.TENSOR_IDS
    hid = syn.device_normal((1, n, D), 3, (5, 0, 0, T["hidden0"]),
                            torch.bfloat16, dev)
    wts = syn.draw_sink_gate_weights(w, 3, 0)
    shape = k.Shape(1, H, G, w.head_dim, n, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    sc = k.Scorer.sink_gate(wts["w"].torch(dev), wts["sinks"].torch(dev),
                            norm=wts["norm"].torch(dev), b=wts["b"].torch(dev))
    k.kve_score(shape, sc, cache, 0, n, hidden=hid)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(n - 64, 536, replace=False),
                                     np.arange(n - 64, n)]))
    idx = torch.from_numpy(rows).to(dev)
    x64 = hid[0].index_select(0, idx).float().cpu().double().numpy()
    ref = oracle_sink_gate_scores(x64[None], wts, H, G)
    got = cache.score[:, :, rows].cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=SINK_GATE_ATOL)
