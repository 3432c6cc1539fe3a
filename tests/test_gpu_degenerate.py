"""Degenerate calls through the boundary: an empty slice, an empty score
range, n_keep == len, compactions with nothing to move. Each must leave
every buffer exactly as the contract in include/kvevict.h says (nothing
written, the identity, the cache bitwise unchanged), on both the small and
the large kernel of each step."""
import numpy as np
import pytest

from kvharness import kve

pytestmark = pytest.mark.gpu


def _cache(k, shape, dev, seed):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    b, H, cap, d = shape.batch, shape.n_kv_heads, shape.capacity, shape.head_dim
    c = k.CacheTensors.empty(shape, dev)
    c.k.copy_(torch.randn((b, H, cap, d), generator=g, device=dev).to(c.k.dtype))
    c.v.copy_(torch.randn((b, H, cap, d), generator=g, device=dev).to(c.v.dtype))
    c.score.copy_(torch.randn((b, H, cap), generator=g, device=dev))
    c.pos.copy_(torch.arange(cap, dtype=torch.int32, device=dev).expand(b, H, cap))
    return c


def _snapshot(c):
    return [t.clone() for t in (c.k, c.v, c.score, c.pos)]


def _unchanged(c, snap):
    import torch
    torch.cuda.synchronize()
    for a, b, name in zip((c.k, c.v, c.score, c.pos), snap,
                          ("k", "v", "score", "pos")):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16
                           else a, b.view(torch.uint8)
                           if b.dtype == torch.bfloat16 else b), name


def test_select_of_an_empty_slice_writes_nothing():
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(2, 3, 1, 128, 64, k.BF16)
    c = _cache(k, shape, dev, 1)
    keep = torch.full((2 * 3 * 4,), -7, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, k.Policy(8, 2, 3, 1), c, 0, 0, keep)
    torch.cuda.synchronize()
    assert bool((keep == -7).all())


@pytest.mark.parametrize("n", [1, 100, 4096, 5000, 50000])
def test_select_with_nothing_to_evict_is_the_identity(n):
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(1, 2, 1, 128, n, k.BF16)
    c = _cache(k, shape, dev, n)
    keep = torch.full((1, 2, n), -7, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, k.Policy(max(n, 8), 2, 3, 1), c, n, n, keep)
    torch.cuda.synchronize()
    ref = torch.arange(n, dtype=torch.int32, device=dev).expand(1, 2, n)
    assert torch.equal(keep, ref)


@pytest.mark.parametrize("n,n_keep", [(100, 60), (3000, 2048), (50000, 39321),
                                      (2048, 2048)])
def test_compact_with_nothing_to_move_leaves_the_cache_unchanged(n, n_keep):
    """Every kept slot lies below n_keep (no holes), or n_keep == len: no
    row may move and nothing at or above n_keep may be touched."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(1, 2, 1, 128, n + 3, k.BF16)
    c = _cache(k, shape, dev, n_keep)
    snap = _snapshot(c)
    keep = torch.arange(n_keep, dtype=torch.int32,
                        device=dev).expand(1, 2, n_keep).contiguous()
    k.kve_compact(shape, c, n, keep, n_keep)
    _unchanged(c, snap)


def test_score_of_an_empty_range_writes_nothing():
    import torch
    k = kve()
    dev = torch.device("cuda")
    shape = k.Shape(2, 2, 1, 128, 256, k.BF16)
    c = _cache(k, shape, dev, 5)
    g = torch.Generator(device=dev).manual_seed(3)
    w1 = (torch.randn((2, 64, 256), generator=g, device=dev) * 0.0625).to(
        torch.bfloat16)
    sc = k.Scorer.mlp(w1, torch.randn((2, 64), generator=g, device=dev))
    snap = _snapshot(c)
    for at in (0, 17, 256):
        k.kve_score(shape, sc, c, at, at)
    _unchanged(c, snap)
