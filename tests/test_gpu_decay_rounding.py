"""Temporal decay ranks by the float32 static priority score - t * log(gamma)
(KVpop Eq. 20, float32 ranking of Appendix F) with the product rounded, then
the difference. Pairs of tokens whose keys tie under those two roundings but
not under one fused multiply-add decide between the two: ties go to the
position rule (the newer token ranks first, the older is evicted first). The
pairs are found on the host from the definition; the GPU's prefill ranks and
its decode selects (register and larger-slice kernels) must follow the
oracle bit for bit."""
import numpy as np
import pytest

import oracle as O
from kvharness import kve

pytestmark = pytest.mark.gpu

LG = float(np.float32(np.log(np.float32(0.9))))


def _two(s, t):
    return np.float32(np.float32(s) - np.float32(np.float32(t) * np.float32(LG)))


def _fused(s, t):
    return np.float32(np.float64(np.float32(s)) -
                      np.float64(np.float32(t)) * np.float64(np.float32(LG)))


def _tied_pairs(count, t_max, seed=1):
    """(t1, s1, t2, s2): equal keys under two roundings, unequal when fused,
    and the fused order would put the newer token first for eviction."""
    rng = np.random.default_rng(seed)
    out, used = [], set()
    while len(out) < count:
        t1, t2 = (int(x) for x in rng.integers(0, t_max, 2))
        if t1 == t2 or t1 in used or t2 in used:
            continue
        s1 = np.float32(rng.standard_normal())
        k1 = _two(s1, t1)
        s2 = np.float32(k1 + np.float32(np.float32(t2) * np.float32(LG)))
        if _two(s2, t2) != k1:
            continue
        f1, f2 = _fused(s1, t1), _fused(s2, t2)
        newer_first = (f1 < f2) if t1 > t2 else (f2 < f1)
        if f1 == f2 or not newer_first:
            continue
        used.update((t1, t2))
        out.append((t1, float(s1), t2, float(s2)))
    return out


def test_prefill_ranks_follow_two_roundings():
    import torch
    k = kve()
    dev = torch.device("cuda")
    n = 2048
    rng = np.random.default_rng(3)
    s = rng.standard_normal(n).astype(np.float32)
    for t1, s1, t2, s2 in _tied_pairs(16, n):
        s[t1], s[t2] = s1, s2
    shape = k.Shape(1, 1, 1, 64, n, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    cache.score[0, 0] = torch.from_numpy(s).to(dev)
    pol = k.Policy(200, 4, 16, 1, log_gamma=torch.tensor([LG], device=dev))
    rank = torch.full((1, 1, n), -7, dtype=torch.int32, device=dev)
    tau = torch.full((1, 1, n), -7, dtype=torch.int32, device=dev)
    k.kve_prefill_select(shape, pol, cache, n, rank, tau)
    torch.cuda.synchronize()
    ref = O.prefill_ranks(s, LG)
    np.testing.assert_array_equal(rank.cpu().numpy()[0, 0], ref)


@pytest.mark.parametrize("n", [1800, 4096, 6000, 50000])
def test_select_evicts_the_older_of_a_two_rounding_tie(n):
    """Every other candidate scores far higher, so the one eviction falls
    inside the tied pair: the older token goes."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    pairs = _tied_pairs(6, min(n, 1800), seed=n)
    H = len(pairs)
    s = np.full((1, H, n), 1.0e4, np.float32)
    for h, (t1, s1, t2, s2) in enumerate(pairs):
        s[0, h, t1], s[0, h, t2] = s1, s2
    pos = np.broadcast_to(np.arange(n), (1, H, n))
    shape = k.Shape(1, H, 1, 64, n, k.BF16)
    cache = k.CacheTensors.empty(shape, dev)
    cache.score.copy_(torch.from_numpy(s).to(dev))
    cache.pos.copy_(torch.from_numpy(pos.astype(np.int32)).to(dev))
    lg = torch.full((H,), LG, device=dev)
    pol = k.Policy(n - 1, 0, 0, 1, log_gamma=lg)
    keep = torch.full((1, H, n - 1), -7, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, pol, cache, n, n - 1, keep)
    got = keep.cpu().numpy()
    for h, (t1, _, t2, _) in enumerate(pairs):
        ref = O.select_keep(s[0, h], pos[0, h], n, n - 1, 0, 0, LG)
        assert min(t1, t2) not in ref and max(t1, t2) in ref
        np.testing.assert_array_equal(got[0, h], ref, err_msg=f"pair {h}")
