"""ForesightKV's stochastic eviction (the Top-K multinomial rule: r draws
without replacement from the 2r lowest-ranked candidates, with probability
proportional to exp(-key)) through the C ABI, against the oracle.

The draw is the Gumbel-top-k one with the noise passed in, so given the same
float32 scores and noise the kept slots are unique: they are compared
bit-exactly, slice by slice.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import (attn_close, kve, oracle_mlp_scores, shape_of,
                       SCORE_ATOL, Tracker)

pytestmark = pytest.mark.gpu


def run_select(b, H, cap, length, n_keep, S, W, scores, pos, noise, lg=None):
    """kve_select_evict with noise; returns the GPU's and the oracle's kept
    slots [b][H][n_keep]."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(b, H, 1, 64, cap, k.F32)
    cache = k.CacheTensors.empty(shape, dev)
    cache.score[:, :, :length] = torch.from_numpy(scores).to(dev)
    cache.pos[:, :, :length] = torch.from_numpy(pos.astype(np.int32)).to(dev)
    gum = torch.zeros((b, H, cap), dtype=torch.float32, device=dev)
    if noise is not None:
        gum[:, :, :length] = torch.from_numpy(noise).to(dev)
    pol = k.Policy(n_keep, S, W, 1,
                   log_gamma=None if lg is None else torch.from_numpy(lg).to(dev),
                   gumbel=gum if noise is not None else None)
    keep = torch.full((b, H, n_keep), -7, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, pol, cache, length, n_keep, keep)
    got = keep.cpu().numpy().astype(np.int64)
    ref = np.empty_like(got)
    for bi in range(b):
        for h in range(H):
            lgh = None if lg is None else float(lg[h])
            if noise is None:
                ref[bi, h] = O.select_keep(scores[bi, h], pos[bi, h], length,
                                           n_keep, S, W, lgh)
            else:
                ref[bi, h] = O.select_keep_stochastic(
                    scores[bi, h], pos[bi, h], length, n_keep, S, W,
                    noise[bi, h], lgh)
    return got, ref


CASES = [
    # b, H, cap, len, n_keep, S, W, score kind, decay
    (2, 3, 300, 300, 200, 4, 16, "ties", False),
    (2, 3, 300, 300, 200, 4, 16, "ties", True),
    (4, 8, 1088, 1088, 1024, 4, 128, "normal", False),   # r = 64, pool 128
    (2, 2, 300, 300, 60, 4, 16, "normal", False),        # pool = candidates
    (1, 2, 700, 613, 600, 0, 0, "ties", False),          # S = W = 0
    (1, 2, 50, 9, 8, 1, 1, "normal", True),              # r = 1
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"b{c[0]}H{c[1]}len{c[3]}keep{c[4]}S{c[5]}W{c[6]}{c[7]}{'-decay' if c[8] else ''}"
    for c in CASES])
def test_stochastic_select_matches_oracle(case):
    b, H, cap, length, n_keep, S, W, kind, decay = case
    print(f"[stochastic] {case}", flush=True)
    rng = np.random.default_rng(length + n_keep)
    if kind == "ties":
        scores = rng.integers(0, 3, (b, H, length)).astype(np.float32)
    else:
        scores = rng.standard_normal((b, H, length)).astype(np.float32)
    pos = np.stack([[rng.permutation(length + 3)[:length] for _ in range(H)]
                    for _ in range(b)])
    lg = (np.log(np.linspace(0.9, 0.999, H))).astype(np.float32) if decay else None
    noise = syn.gumbel_noise(rng, (b, H, length))
    got, ref = run_select(b, H, cap, length, n_keep, S, W, scores, pos, noise,
                          lg)
    np.testing.assert_array_equal(got, ref)
    # zero noise: the deterministic rule, on the GPU and in the oracle
    got0, _ = run_select(b, H, cap, length, n_keep, S, W, scores, pos,
                         np.zeros_like(noise), lg)
    det, _ = run_select(b, H, cap, length, n_keep, S, W, scores, pos, None, lg)
    np.testing.assert_array_equal(got0, det)


def test_stochastic_select_tied_sums():
    """Integer scores and integer noise: many perturbed sums are equal, so
    the position order decides inside the draw."""
    b, H, length, n_keep = 2, 4, 400, 250
    rng = np.random.default_rng(5)
    scores = rng.integers(-2, 3, (b, H, length)).astype(np.float32)
    noise = rng.integers(-2, 3, (b, H, length)).astype(np.float32)
    pos = np.stack([[rng.permutation(length) for _ in range(H)]
                    for _ in range(b)])
    got, ref = run_select(b, H, length, length, n_keep, 4, 8, scores, pos,
                          noise)
    np.testing.assert_array_equal(got, ref)


def test_stochastic_select_full_size():
    """Batch 96 x 8 KV heads at B + L = 1152 entries (r = 128, pool 256), and
    the 131072-token one-shot compression to B = 39321 of 8 KV heads (pool
    = every candidate)."""
    print("[stochastic] full size", flush=True)
    rng = np.random.default_rng(9)
    b, H, length = 96, 8, 1152
    scores = rng.standard_normal((b, H, length)).astype(np.float32)
    pos = np.stack([[rng.permutation(9000)[:length] for _ in range(H)]
                    for _ in range(b)])
    noise = syn.gumbel_noise(rng, (b, H, length))
    got, ref = run_select(b, H, length, length, 1024, 4, 128, scores, pos,
                          noise)
    np.testing.assert_array_equal(got, ref)
    n = 131072
    scores = rng.standard_normal((1, 8, n)).astype(np.float32)
    pos = np.broadcast_to(np.arange(n), (1, 8, n)).copy()
    noise = syn.gumbel_noise(rng, (1, 8, n))
    got, ref = run_select(1, 8, n, n, 39321, 4, 512, scores, pos, noise)
    np.testing.assert_array_equal(got, ref)


def test_stochastic_step_end_to_end():
    """kve_step with fresh noise before every step: the MLP-scored Qwen3-4B
    layer shapes at batch 2, a 2048-token prompt compressed to B = 512
    (deterministically), W = 64, L = 32, 100 steps (three stochastic
    evictions); retained sets against the oracle loop drawing with the same
    noise, attention over them every step."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(2, batch=2, n0=2048, budget=512, window=64, evict_len=32,
                     steps=100)
    seed, layer = 0, 0
    ctx = syn.initial_context(w, seed, layer)
    wts = syn.draw_mlp_weights(w, seed, layer, biases=True)
    s0 = oracle_mlp_scores(ctx["k0"].f64, ctx["v0"].f64, wts, w.act)
    sc = k.Scorer.mlp(wts["w1"].torch(dev), wts["w2"].torch(dev),
                      wts["b1"].torch(dev), wts["b2"].torch(dev))
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    tr = Tracker(w, ctx["k0"].f64, ctx["v0"].f64, s0, pol_o)
    shape = shape_of(w)
    gum = torch.zeros((w.batch, w.n_kv, w.capacity), dtype=torch.float32,
                      device=dev)
    pol_det = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len, gumbel=gum)
    cache = k.CacheTensors.empty(shape, dev)
    cache.k[:, :, :w.n0] = ctx["k0"].torch(dev)
    cache.v[:, :, :w.n0] = ctx["v0"].torch(dev)
    cache.pos[:, :, :w.n0] = torch.arange(w.n0, dtype=torch.int32, device=dev)
    keep = torch.zeros((w.batch, w.n_kv, w.capacity), dtype=torch.int32,
                       device=dev)
    ws = k.alloc_workspace(shape, w.capacity, dev)
    k.kve_score(shape, sc, cache, 0, w.n0)
    tr.prefill()
    k.kve_select_evict(shape, pol_det, cache, w.n0, w.budget, keep)
    k.kve_compact(shape, cache, w.n0, keep, w.budget)
    tr.check_and_sync(cache.pos[:, :, :w.budget].cpu().numpy().astype(np.int64))
    state = k.DecodeState(w.budget, w.budget, w.n0)
    out = torch.zeros((w.batch, w.n_q, w.head_dim), device=dev)
    lse = torch.zeros((w.batch, w.n_q), device=dev)
    rng = np.random.default_rng(17)
    evictions = 0
    for i in range(w.steps):
        st = syn.step_inputs(w, seed, layer, i)
        noise = syn.gumbel_noise(rng, (w.batch, w.n_kv, w.capacity))
        gum.copy_(torch.from_numpy(noise).to(dev))
        sn = oracle_mlp_scores(st["k_new"].f64[:, :, None],
                               st["v_new"].f64[:, :, None], wts, w.act)[:, :, 0]
        k.kve_step(shape, pol, sc, cache, state, st["k_new"].torch(dev),
                   st["v_new"].torch(dev), st["q"].torch(dev), out, lse, keep,
                   ws)
        tr.step(w.n0 + i, st["k_new"].f64, st["v_new"].f64, sn, gumbel=noise)
        evictions += state.evicted
        torch.cuda.synchronize()
        gpu_pos = cache.pos[:, :, :state.len].cpu().numpy().astype(np.int64)
        assert state.len == tr.lay.n
        if state.evicted:
            # The draw has no tolerance band: the sets must be equal.
            np.testing.assert_array_equal(np.sort(gpu_pos, axis=2),
                                          np.sort(tr.lay.pos, axis=2))
            gs = cache.score[:, :, :state.len].cpu().numpy()
            ref = np.take_along_axis(tr.S, gpu_pos, axis=2)
            np.testing.assert_allclose(gs, ref, rtol=0, atol=SCORE_ATOL)
        tr.check_and_sync(gpu_pos)
        ref_out, _ = tr.lay.attend(st["q"].f64)
        attn_close(out.cpu().double().numpy(), ref_out, f"step {i}")
    assert evictions == 3
