"""The library keeps no state between calls, so independent layers stepped
on two streams at once give the same bits as the same steps run one layer
after the other on one stream: caches, kept slots and every step's output
and log-sum-exp. Each layer has its own workspace, and the split-K shape
(batch 4, 8 KV heads, long slices) uses it. Both streams are created with
the default priority."""
import numpy as np
import pytest

from kvharness import kve

pytestmark = pytest.mark.gpu

BATCH, H, G, D = 4, 8, 4, 128
B, S, W, L = 1536, 4, 64, 64
STEPS = 200  # three evictions per layer


def _layer(k, shape, dev, seed):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    cap = shape.capacity
    c = k.CacheTensors.empty(shape, dev)
    c.k.copy_(torch.randn((BATCH, H, cap, D), generator=g, device=dev).to(
        torch.bfloat16))
    c.v.copy_(torch.randn((BATCH, H, cap, D), generator=g, device=dev).to(
        torch.bfloat16))
    c.score.copy_(torch.randn((BATCH, H, cap), generator=g, device=dev))
    c.pos.copy_(torch.arange(cap, dtype=torch.int32, device=dev).expand(
        BATCH, H, cap))
    c.pos[:, :, B:] = -1
    return c


def _clone(k, c):
    return k.CacheTensors(c.k.clone(), c.v.clone(), c.score.clone(),
                          c.pos.clone())


def _inputs(dev, seed):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    kn = torch.randn((STEPS, BATCH, H, D), generator=g, device=dev).to(
        torch.bfloat16)
    vn = torch.randn((STEPS, BATCH, H, D), generator=g, device=dev).to(
        torch.bfloat16)
    q = torch.randn((STEPS, BATCH, H * G, D), generator=g, device=dev).to(
        torch.bfloat16)
    return kn, vn, q


def test_two_streams_equal_one_stream():
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(BATCH, H, G, D, B + L, k.BF16)
    pol = k.Policy(B, S, W, L)
    gw = torch.Generator(device=dev).manual_seed(5)
    w1 = (torch.randn((H, 64, 2 * D), generator=gw, device=dev) *
          (2 * D) ** -0.5).to(torch.bfloat16)
    sc = k.Scorer.mlp(w1, torch.randn((H, 64), generator=gw, device=dev))
    base = [_layer(k, shape, dev, 11 + i) for i in range(2)]
    inputs = [_inputs(dev, 21 + i) for i in range(2)]

    def run(streams):
        caches = [_clone(k, c) for c in base]
        states = [k.DecodeState(B, B, B) for _ in range(2)]
        outs = [torch.empty((STEPS, BATCH, H * G, D), device=dev)
                for _ in range(2)]
        lses = [torch.empty((STEPS, BATCH, H * G), device=dev)
                for _ in range(2)]
        keeps = [torch.full((BATCH, H, B), -1, dtype=torch.int32, device=dev)
                 for _ in range(2)]
        wss = [k.alloc_workspace(shape, shape.capacity, dev) for _ in range(2)]
        torch.cuda.synchronize()
        evictions = [0, 0]

        def one(i, s):
            kn, vn, q = inputs[i]
            out = outs[i][s]
            lse = lses[i][s]
            k.kve_step(shape, pol, sc, caches[i], states[i], kn[s], vn[s],
                       q[s], out, lse, keeps[i], wss[i], stream=streams[i])
            evictions[i] += states[i].evicted

        if streams[0] is streams[1]:
            for i in range(2):
                for s in range(STEPS):
                    one(i, s)
        else:
            for s in range(STEPS):
                for i in range(2):
                    one(i, s)
        torch.cuda.synchronize()
        assert evictions == [3, 3]
        return caches, outs, lses, keeps

    main = torch.cuda.current_stream()
    seq = run([main, main])
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    par = run([s0, s1])
    for i in range(2):
        a, b = seq[0][i], par[0][i]
        for x, y, name in ((a.k, b.k, "k"), (a.v, b.v, "v"),
                           (a.score, b.score, "score"), (a.pos, b.pos, "pos")):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16
                               else x.view(torch.int32),
                               y.view(torch.int16) if y.dtype == torch.bfloat16
                               else y.view(torch.int32)), f"layer {i} {name}"
        assert torch.equal(seq[1][i].view(torch.int32), par[1][i].view(torch.int32))
        assert torch.equal(seq[2][i].view(torch.int32), par[2][i].view(torch.int32))
        assert torch.equal(seq[3][i], par[3][i])
