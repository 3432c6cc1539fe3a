"""kve_step_noalloc, the decode step for callers that cannot allocate: its
split-K partials live in the library's per-GPU scratch array instead of a
caller workspace. It runs the same kernels with the same split plan as
kve_step, so every output, the whole cache and the kept slots must be
bitwise equal to kve_step's with a torch-allocated workspace. Two workloads
in a row, the second smaller (both split, so both use the scratch array),
each over three steps: a fused append, a scoring + eviction step and a fused
append after it."""
import numpy as np
import pytest

from kvharness import kve

pytestmark = pytest.mark.gpu


def _setup(k, dev, batch, H, G, D, B, L, S, W, seed):
    import torch
    gen = torch.Generator().manual_seed(seed)
    cap = B + L
    shape = k.Shape(batch, H, G, D, cap, k.BF16)
    pol = k.Policy(B, S, W, L)
    n0 = B + L - 2
    caches = []
    kv = [torch.randn((batch, H, cap, D), generator=gen).to(torch.bfloat16)
          for _ in range(2)]
    sc = torch.randn((batch, H, cap), generator=gen)
    for _ in range(2):
        c = k.CacheTensors.empty(shape, dev)
        c.k.copy_(kv[0].to(dev))
        c.v.copy_(kv[1].to(dev))
        c.score.copy_(sc.to(dev))
        c.pos.copy_(torch.arange(cap, dtype=torch.int32).expand(batch, H, cap)
                    .to(dev))
        caches.append(c)
    w1 = (torch.randn((H, 64, 2 * D), generator=gen) * (2 * D) ** -0.5
          ).to(torch.bfloat16).to(dev)
    w2 = (torch.randn((H, 64), generator=gen) * 64 ** -0.5).to(dev)
    scorer = k.Scorer.mlp(w1, w2)
    steps = []
    for _ in range(3):
        steps.append(tuple(
            torch.randn(s, generator=gen).to(torch.bfloat16).to(dev)
            for s in ((batch, H, D), (batch, H, D), (batch, H * G, D))))
    return shape, pol, scorer, caches, n0, steps


@pytest.mark.parametrize("seed", [0])
def test_noalloc_step_equals_step_with_workspace(seed):
    import torch
    k = kve()
    dev = torch.device("cuda:0")
    # the batch-8 Qwen3-4B layer at B = 2048 (64 slices, split in 4), then a
    # smaller G = 5 layer (16 slices, split in several)
    for case in [(8, 8, 4, 128, 2048, 256, 4, 256),
                 (2, 8, 5, 128, 512, 64, 4, 64)]:
        print(f"[noalloc] case {case}", flush=True)
        batch, H, G, D, B, L, S, W = case
        shape, pol, scorer, caches, n0, steps = _setup(
            k, dev, batch, H, G, D, B, L, S, W, seed)
        ws = k.alloc_workspace(shape, shape.capacity, dev)
        states = [k.DecodeState(n0, B, n0) for _ in range(2)]
        for i, (kn, vn, q) in enumerate(steps):
            outs, lses, keeps = [], [], []
            for j in range(2):
                out = torch.full((batch, H * G, D), float("nan"), device=dev)
                lse = torch.full((batch, H * G), float("nan"), device=dev)
                keep = torch.full((batch, H, B), -1, dtype=torch.int32,
                                  device=dev)
                if j == 0:
                    k.kve_step(shape, pol, scorer, caches[j], states[j], kn,
                               vn, q, out, lse, keep, ws)
                else:
                    k.kve_step_noalloc(shape, pol, scorer, caches[j],
                                       states[j], kn, vn, q, out, lse, keep)
                outs.append(out)
                lses.append(lse)
                keeps.append(keep)
            torch.cuda.synchronize()
            a, b = states
            assert (a.len, a.scored_upto, a.next_position, a.evicted) == \
                (b.len, b.scored_upto, b.next_position, b.evicted), i
            assert a.evicted == (1 if i == 1 else 0), i
            assert torch.equal(outs[0], outs[1]), (case, i)
            assert torch.equal(lses[0], lses[1]), (case, i)
            assert not torch.isnan(outs[1]).any(), (case, i)
            assert torch.equal(keeps[0], keeps[1]), (case, i)
            for name in ("k", "v", "score", "pos"):
                x, y = getattr(caches[0], name), getattr(caches[1], name)
                assert torch.equal(x.view(torch.int16) if x.dtype ==
                                   torch.bfloat16 else x,
                                   y.view(torch.int16) if y.dtype ==
                                   torch.bfloat16 else y), (case, i, name)
