"""Full-size parity in the launch configuration the benchmark times.

One layer of the batch-96 Qwen3-4B-shaped workload (8 KV heads, 32 query
heads, head_dim 128, bf16; an 8192-token prompt scored, selected and
compacted to B = 1024, then L = 128 periodic eviction) runs through the
same calls as bench.py (library prompt compression, then LayerStep per
decode step). The inputs come from the synthetic generator on the device.
For sampled (batch, KV head) slices the float64 oracle replays the whole
history from those same inputs, independently of the GPU state, and every
step is checked: retained positions (equal except at score ties within
1e-3 of the cut), scores of the retained entries (1e-3 abs) and the G query
heads' attention outputs (2e-3 * max|out|).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import ATTN_RTOL, SCORE_ATOL, kve

pytestmark = pytest.mark.gpu

SAMPLED = {4: [(0, 0), (17, 3), (50, 5), (95, 7)],
           3: [(0, 1), (5, 6), (7, 7)]}
STEPS = {4: 256, 3: 512}


class SliceOracle:
    """The oracle's view of one (batch, KV head) slice, given the float32
    scores the oracle computed for its tokens."""

    def __init__(self, k0, v0, s0, policy, group):
        self.score_by_pos = {t: float(s0[t]) for t in range(k0.shape[0])}
        self.lay = O.OracleLayer(k0[None, None], v0[None, None],
                                 s0[None, None], policy, group)
        self.cut = None
        self.policy = policy
        if self.lay.prefill_compress() is not None:
            self._cut()

    def _cut(self):
        """Lowest kept score among the eligible entries after an eviction."""
        p = self.policy
        m = O.eligible_mask(self.lay.pos[0, 0], p.sinks, p.window)
        self.cut = float(self.lay.score[0, 0][m].min())

    def step(self, pos, k, v, s_new, q):
        self.score_by_pos[pos] = float(s_new)
        self.lay.append(k[None, None], v[None, None],
                        np.array([[s_new]], np.float32))
        if self.lay.maybe_evict() is not None:
            self._cut()
        out, _ = self.lay.attend(q[None])
        return out[0]

    def sync_to(self, gpu_pos, K_by_pos, V_by_pos):
        """Adopt the GPU's retained entries and slot order after a tolerated
        tie flip (different entries kept at the cut also place the moved
        entries differently)."""
        o = self.lay.pos[0, 0]
        diff = set(gpu_pos.tolist()) ^ set(o.tolist())
        for t in diff:
            assert abs(self.score_by_pos[t] - self.cut) <= SCORE_ATOL, \
                f"token {t} differs beyond the tie band"
        self.lay.pos = gpu_pos[None, None].astype(np.int64)
        self.lay.K = np.stack([K_by_pos[t] for t in gpu_pos])[None, None]
        self.lay.V = np.stack([V_by_pos[t] for t in gpu_pos])[None, None]
        self.lay.score = np.array([self.score_by_pos[t] for t in gpu_pos],
                                  np.float32)[None, None]


def mlp_relu(k, v, w1, w2):
    return O.mlp_score(k, v, w1, np.zeros(w1.shape[0]), w2, 0.0, "relu")


def _host64(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("cfg", [4, 3], ids=["b96-B1024-L128", "b8-B2048-L256"])
def test_layer_sampled_slices_every_step(cfg):
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(cfg, layers=1, steps=STEPS[cfg])
    sampled = SAMPLED[cfg]
    T = syn.TENSOR_IDS
    b, H, G, d = w.batch, w.n_kv, w.group, w.head_dim
    seed, cfg, layer = 0, w.cfg_id, 0
    dn = syn.device_normal
    print(f"[fullsize] {w.name} batch={b} n0={w.n0} B={w.budget} "
          f"steps={w.steps}", flush=True)
    w1 = dn((H, w.hidden, 2 * d), seed, (cfg, layer, 0, T["w1"]),
            torch.bfloat16, dev, scale=(2 * d) ** -0.5)
    w2 = dn((H, w.hidden), seed, (cfg, layer, 0, T["w2"]), torch.float32,
            dev, scale=w.hidden ** -0.5)
    k0 = dn((b, H, w.n0, d), seed, (cfg, layer, 0, T["k0"]), torch.bfloat16,
            dev)
    v0 = dn((b, H, w.n0, d), seed, (cfg, layer, 0, T["v0"]), torch.bfloat16,
            dev)
    kn = dn((w.steps, b, H, d), seed, (cfg, layer, 1, T["k_new"]),
            torch.bfloat16, dev)
    vn = dn((w.steps, b, H, d), seed, (cfg, layer, 1, T["v_new"]),
            torch.bfloat16, dev)
    qs = dn((w.steps, b, H * G, d), seed, (cfg, layer, 1, T["q"]),
            torch.bfloat16, dev)

    # Oracle side: sampled slices, from the same generated inputs.
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    w1h, w2h = _host64(w1), _host64(w2)
    oracles, kpos, vpos = {}, {}, {}
    for (bi, h) in sampled:
        k0s, v0s = _host64(k0[bi, h]), _host64(v0[bi, h])
        s0 = O.score_to_f32(mlp_relu(k0s, v0s, w1h[h], w2h[h]))
        oracles[(bi, h)] = SliceOracle(k0s, v0s, s0, pol_o, G)
        kpos[(bi, h)] = {t: k0s[t] for t in range(w.n0)}
        vpos[(bi, h)] = {t: v0s[t] for t in range(w.n0)}
    kn_h = {s: _host64(kn[:, s[0], s[1]]) for s in sampled}
    vn_h = {s: _host64(vn[:, s[0], s[1]]) for s in sampled}
    q_h = {s: _host64(qs[:, s[0], s[1] * G:(s[1] + 1) * G]) for s in sampled}

    # HIP path: the benchmark's calls.
    pre = k.Shape(b, H, G, d, w.n0, k.BF16)
    shape = k.Shape(b, H, G, d, w.budget + w.evict_len, k.BF16)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    sc = k.Scorer.mlp(w1, w2)
    scratch = k.CacheTensors(k0, v0, torch.empty((b, H, w.n0), device=dev),
                             torch.arange(w.n0, dtype=torch.int32,
                                          device=dev).repeat(b, H, 1))
    keep_pre = torch.empty((b, H, w.budget), dtype=torch.int32, device=dev)
    k.kve_score(pre, sc, scratch, 0, w.n0)
    k.kve_select_evict(pre, pol, scratch, w.n0, w.budget, keep_pre)
    k.kve_compact(pre, scratch, w.n0, keep_pre, w.budget)
    cache = k.CacheTensors.empty(shape, dev)
    B = w.budget
    cache.k[:, :, :B].copy_(k0[:, :, :B])
    cache.v[:, :, :B].copy_(v0[:, :, :B])
    cache.score[:, :, :B].copy_(scratch.score[:, :, :B])
    cache.pos[:, :, :B].copy_(scratch.pos[:, :, :B])
    del scratch, k0, v0
    ws = k.alloc_workspace(shape, shape.capacity, dev)
    state = k.DecodeState(B, B, w.n0)
    run = k.LayerStep(shape, pol, sc, cache, state, ws)
    out = torch.empty((b, H * G, d), dtype=torch.float32, device=dev)
    keep = torch.empty((b, H, shape.capacity), dtype=torch.int32, device=dev)

    evictions, worst = 0, 0.0
    for i in range(w.steps):
        evictions += run(kn[i], vn[i], qs[i], out, None, keep)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        n = state.len
        for s in sampled:
            bi, h = s
            o = oracles[s]
            pos_i = w.n0 + i
            kpos[s][pos_i], vpos[s][pos_i] = kn_h[s][i], vn_h[s][i]
            s_new = O.score_to_f32(mlp_relu(kn_h[s][i][None], vn_h[s][i][None],
                                            w1h[h], w2h[h]))[0]
            ref = o.step(pos_i, kn_h[s][i], vn_h[s][i], s_new, q_h[s][i])
            # slot by slot: both sides place entries the same way
            gpos = cache.pos[bi, h, :n].cpu().numpy().astype(np.int64)
            assert n == o.lay.n, f"step {i}: count {n} != {o.lay.n}"
            if not np.array_equal(gpos, o.lay.pos[0, 0]):
                o.sync_to(gpos, kpos[s], vpos[s])
                ref = o.lay.attend(q_h[s][i][None])[0][0]
            g = got[bi, h * G:(h + 1) * G]
            rel = np.abs(g - ref).max() / np.abs(ref).max()
            worst = max(worst, rel)
            assert rel <= ATTN_RTOL, f"step {i} slice {s}: rel err {rel:.2e}"
            if state.evicted:
                gs = cache.score[bi, h, :n].cpu().numpy()
                ref_s = np.array([o.score_by_pos[t] for t in gpos])
                np.testing.assert_allclose(gs, ref_s, rtol=0, atol=SCORE_ATOL)
        if i % 64 == 63:
            print(f"[fullsize] step {i + 1}: worst rel err {worst:.2e}",
                  flush=True)
    assert evictions == w.steps // w.evict_len  # every L-th step reaches B + L
    assert state.len == B


def _gate_scores_chunked(hidden_bits, w, chunk=8192):
    """Oracle gate scores of every token, from bf16 hidden states held as
    raw bits on the host, converted to float64 chunk by chunk."""
    out = np.empty(hidden_bits.shape[0], np.float32)
    for r0 in range(0, hidden_bits.shape[0], chunk):
        x = syn.bf16_bits_to_f32(hidden_bits[r0:r0 + chunk]).astype(np.float64)
        out[r0:r0 + chunk] = O.score_to_f32(O.gate_score(x, w))
    return out


def test_gate_131k_prompt_sampled_heads():
    """Qwen2.5-14B-shaped layer (8 KV heads, 40 query heads, d 128, bf16):
    a 131072-token prompt gated per KV head from 5120-dim hidden states,
    compressed once to 30% (B = 39321, S = 4, W = 512), then L = 64
    buffered gate scoring with periodic eviction."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    w = syn.workload(5, layers=1, steps=128)
    T = syn.TENSOR_IDS
    b, H, G, d, D = w.batch, w.n_kv, w.group, w.head_dim, w.hidden
    seed, cfg, layer = 0, w.cfg_id, 0
    dn = syn.device_normal
    print(f"[fullsize] {w.name} n0={w.n0} B={w.budget} L={w.evict_len} "
          f"steps={w.steps}", flush=True)
    gw = dn((H, D), seed, (cfg, layer, 0, T["gate_w"]), torch.bfloat16, dev,
            scale=D ** -0.5)
    hid0 = dn((b, w.n0, D), seed, (cfg, layer, 0, T["hidden0"]),
              torch.bfloat16, dev)
    k0 = dn((b, H, w.n0, d), seed, (cfg, layer, 0, T["k0"]), torch.bfloat16,
            dev)
    v0 = dn((b, H, w.n0, d), seed, (cfg, layer, 0, T["v0"]), torch.bfloat16,
            dev)
    kn = dn((w.steps, b, H, d), seed, (cfg, layer, 1, T["k_new"]),
            torch.bfloat16, dev)
    vn = dn((w.steps, b, H, d), seed, (cfg, layer, 1, T["v_new"]),
            torch.bfloat16, dev)
    qs = dn((w.steps, b, H * G, d), seed, (cfg, layer, 1, T["q"]),
            torch.bfloat16, dev)
    hn = dn((w.steps, b, D), seed, (cfg, layer, 1, T["hidden_new"]),
            torch.bfloat16, dev)

    sampled = [(0, 0), (0, 6)]
    pol_o = O.Policy(w.budget, w.sinks, w.window, w.evict_len)
    gwh = _host64(gw)
    hbits = hid0[0].cpu().view(torch.int16).numpy().view(np.uint16)
    oracles, kpos, vpos = {}, {}, {}
    for (bi, h) in sampled:
        k0s, v0s = _host64(k0[bi, h]), _host64(v0[bi, h])
        s0 = _gate_scores_chunked(hbits, gwh[h])
        oracles[(bi, h)] = SliceOracle(k0s, v0s, s0, pol_o, G)
        kpos[(bi, h)] = {t: k0s[t] for t in range(w.n0)}
        vpos[(bi, h)] = {t: v0s[t] for t in range(w.n0)}
    del hbits
    kn_h = {s: _host64(kn[:, s[0], s[1]]) for s in sampled}
    vn_h = {s: _host64(vn[:, s[0], s[1]]) for s in sampled}
    q_h = {s: _host64(qs[:, s[0], s[1] * G:(s[1] + 1) * G]) for s in sampled}
    hn_h = _host64(hn[:, 0])
    print("[fullsize] oracle prompt compression done", flush=True)

    pre = k.Shape(b, H, G, d, w.n0, k.BF16)
    shape = k.Shape(b, H, G, d, w.budget + w.evict_len, k.BF16)
    pol = k.Policy(w.budget, w.sinks, w.window, w.evict_len)
    sc = k.Scorer.gate(gw)
    scratch = k.CacheTensors(k0, v0, torch.empty((b, H, w.n0), device=dev),
                             torch.arange(w.n0, dtype=torch.int32,
                                          device=dev).repeat(b, H, 1))
    keep_pre = torch.empty((b, H, w.budget), dtype=torch.int32, device=dev)
    k.kve_score(pre, sc, scratch, 0, w.n0, hidden=hid0)
    k.kve_select_evict(pre, pol, scratch, w.n0, w.budget, keep_pre)
    k.kve_compact(pre, scratch, w.n0, keep_pre, w.budget)
    cache = k.CacheTensors.empty(shape, dev)
    B = w.budget
    cache.k[:, :, :B].copy_(k0[:, :, :B])
    cache.v[:, :, :B].copy_(v0[:, :, :B])
    cache.score[:, :, :B].copy_(scratch.score[:, :, :B])
    cache.pos[:, :, :B].copy_(scratch.pos[:, :, :B])
    del scratch, k0, v0, hid0
    ws = k.alloc_workspace(shape, shape.capacity, dev)
    state = k.DecodeState(B, B, w.n0)
    run = k.LayerStep(shape, pol, sc, cache, state, ws)
    out = torch.empty((b, H * G, d), dtype=torch.float32, device=dev)
    keep = torch.empty((b, H, shape.capacity), dtype=torch.int32, device=dev)
    hbuf = torch.zeros((b, w.evict_len, D), dtype=torch.bfloat16, device=dev)

    evictions, worst = 0, 0.0
    for i in range(w.steps):
        evictions += run(kn[i], vn[i], qs[i], out, None, keep,
                         hidden_new=hn[i], hidden_buf=hbuf)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        n = state.len
        for s in sampled:
            bi, h = s
            o = oracles[s]
            pos_i = w.n0 + i
            kpos[s][pos_i], vpos[s][pos_i] = kn_h[s][i], vn_h[s][i]
            s_new = O.score_to_f32(O.gate_score(hn_h[i], gwh[h]))
            ref = o.step(pos_i, kn_h[s][i], vn_h[s][i], s_new, q_h[s][i])
            # slot by slot: both sides place entries the same way
            gpos = cache.pos[bi, h, :n].cpu().numpy().astype(np.int64)
            assert n == o.lay.n, f"step {i}: count {n} != {o.lay.n}"
            if not np.array_equal(gpos, o.lay.pos[0, 0]):
                o.sync_to(gpos, kpos[s], vpos[s])
                ref = o.lay.attend(q_h[s][i][None])[0][0]
            g = got[bi, h * G:(h + 1) * G]
            rel = np.abs(g - ref).max() / np.abs(ref).max()
            worst = max(worst, rel)
            assert rel <= ATTN_RTOL, f"step {i} slice {s}: rel err {rel:.2e}"
            if state.evicted:
                gs = cache.score[bi, h, :n].cpu().numpy()
                ref_s = np.array([o.score_by_pos[t] for t in gpos])
                np.testing.assert_allclose(gs, ref_s, rtol=0, atol=SCORE_ATOL)
        if i % 64 == 63:
            print(f"[fullsize] step {i + 1}: worst rel err {worst:.2e}",
                  flush=True)
    assert evictions == w.steps // w.evict_len
    assert state.len == B
