"""a3 select and a4 compact: bit-exact against the oracle when both sides
are given the same float32 scores and positions, including every kind of
tie and caches whose slot order is not position order."""
import numpy as np
import pytest

import oracle as O
from kvharness import kve

pytestmark = pytest.mark.gpu


def _scores(rng, pattern, shape):
    if pattern == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if pattern == "ties3":
        return rng.choice(np.array([-1.0, 0.5, 2.0], np.float32), size=shape)
    if pattern == "const":
        return np.full(shape, 0.25, np.float32)
    if pattern == "zeros":  # mix of -0.0 and +0.0 ranks as equal
        return np.where(rng.random(shape) < 0.5, np.float32(-0.0),
                        np.float32(0.0)).astype(np.float32)
    if pattern == "sigmoid":  # gate outputs: values in (0, 1), some ties
        x = 1.0 / (1.0 + np.exp(-rng.standard_normal(shape) * 4))
        x = np.round(x, 3)
        return x.astype(np.float32)
    if pattern == "wide":  # spans many binades, negative and positive
        return (rng.standard_normal(shape) * 10.0 ** rng.integers(
            -30, 30, shape)).astype(np.float32)
    raise ValueError(pattern)


SELECT_CASES = [
    # S, W, len, n_keep, batch, H
    (4, 64, 193, 192, 1, 2),       # L = 1 boundary eviction
    (4, 64, 512, 192, 1, 2),       # prefill compression
    (4, 128, 1152, 1024, 2, 8),    # L = 128
    (4, 256, 2304, 2048, 1, 8),    # L = 256
    (0, 0, 50, 10, 1, 3),          # no protected slots
    (2, 3, 10, 5, 2, 2),           # k = 0: sinks + window only
    (3, 5, 40, 40, 1, 2),          # nothing to evict
    (4, 512, 39385, 39321, 1, 8),  # Qwen2.5-14B decode eviction
    # keys held in LDS up to 40000 entries (few slices), global beyond
    (4, 128, 40000, 30000, 1, 2),
    (4, 128, 40001, 30000, 1, 2),
    (4, 64, 4096, 1024, 32, 8),    # 256 slices, LDS keys
]


def _cache_for_scores(k, shape, scores_np, pos_np, dev):
    import torch
    tiny = torch.zeros(1, device=dev)
    c = k.CacheTensors(tiny, tiny, torch.from_numpy(scores_np).to(dev),
                       torch.from_numpy(pos_np.astype(np.int32)).to(dev))
    return c


def _positions(rng, B, H, cap, n, order):
    """Positions 0..n-1 per slice (slots past n: -1), in slot order or
    shuffled (a cache whose evictions filled holes from the end)."""
    pos = np.full((B, H, cap), -1, np.int64)
    for b in range(B):
        for h in range(H):
            pos[b, h, :n] = (np.arange(n) if order == "sorted"
                             else rng.permutation(n))
    return pos


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("pattern", ["normal", "ties3", "const", "zeros",
                                     "sigmoid", "wide"])
@pytest.mark.parametrize("case", SELECT_CASES,
                         ids=[f"S{c[0]}W{c[1]}n{c[2]}k{c[3]}"
                              for c in SELECT_CASES])
def test_select_bit_exact(case, pattern, order):
    import torch
    k = kve()
    S, W, n, nk, B, H = case
    print(f"[select] {case} {pattern} {order}", flush=True)
    cap = n + 7
    rng = np.random.default_rng(n * 31 + nk)
    sc = _scores(rng, pattern, (B, H, cap))
    pos = _positions(rng, B, H, cap, n, order)
    shape = k.Shape(B, H, 1, 128, cap, k.BF16)
    pol = k.Policy(max(nk, S + W), S, W, 1)
    dev = torch.device("cuda")
    cache = _cache_for_scores(k, shape, sc, pos, dev)
    keep = torch.full((B, H, nk), -1, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, pol, cache, n, nk, keep)
    got = keep.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = O.select_keep(sc[b, h, :n], pos[b, h, :n], n, nk, S, W)
            np.testing.assert_array_equal(got[b, h], ref,
                                          err_msg=f"slice {b},{h}")


DECAY_CASES = [
    # S, W, len, n_keep, batch, H
    (4, 64, 193, 192, 1, 2),
    (4, 128, 1152, 1024, 2, 8),
    (4, 512, 39385, 39321, 1, 8),
    (2, 3, 40, 20, 1, 3),
]


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("pattern", ["normal", "ties3", "const"])
@pytest.mark.parametrize("case", DECAY_CASES,
                         ids=[f"S{c[0]}W{c[1]}n{c[2]}k{c[3]}"
                              for c in DECAY_CASES])
def test_select_with_decay_bit_exact(case, pattern, order):
    """Temporal decay (KVpop Eq. 20): ranking by score - pos * log(gamma_h),
    per KV head, in float32 on both sides."""
    import torch
    k = kve()
    S, W, n, nk, B, H = case
    print(f"[select-decay] {case} {pattern} {order}", flush=True)
    cap = n + 5
    rng = np.random.default_rng(n * 7 + nk)
    sc = _scores(rng, pattern, (B, H, cap))
    pos = _positions(rng, B, H, cap, n, order)
    lg = np.log(np.linspace(0.9, 0.999999, H)).astype(np.float32)
    shape = k.Shape(B, H, 1, 128, cap, k.BF16)
    dev = torch.device("cuda")
    pol = k.Policy(max(nk, S + W), S, W, 1,
                   log_gamma=torch.from_numpy(lg).to(dev))
    cache = _cache_for_scores(k, shape, sc, pos, dev)
    keep = torch.full((B, H, nk), -1, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, pol, cache, n, nk, keep)
    got = keep.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = O.select_keep(sc[b, h, :n], pos[b, h, :n], n, nk, S, W,
                                float(lg[h]))
            np.testing.assert_array_equal(got[b, h], ref,
                                          err_msg=f"slice {b},{h}")


def test_select_one_shot_compression_131k():
    """Qwen2.5-14B prompt of 131072 tokens cut to a 30% budget in one go."""
    import torch
    k = kve()
    S, W, n, nk, B, H = 4, 512, 131072, 39321, 1, 8
    rng = np.random.default_rng(99)
    sc = _scores(rng, "sigmoid", (B, H, n))
    pos = _positions(rng, B, H, n, n, "sorted")
    shape = k.Shape(B, H, 5, 128, n, k.BF16)
    pol = k.Policy(nk, S, W, 64)
    dev = torch.device("cuda")
    cache = _cache_for_scores(k, shape, sc, pos, dev)
    keep = torch.full((B, H, nk), -1, dtype=torch.int32, device=dev)
    k.kve_select_evict(shape, pol, cache, n, nk, keep)
    got = keep.cpu().numpy()
    for h in range(H):
        ref = O.select_keep(sc[0, h], pos[0, h], n, nk, S, W)
        np.testing.assert_array_equal(got[0, h], ref)


def _keep_lists(rng, n, nk, S, W, kind):
    if kind == "select":
        sc = rng.standard_normal(n).astype(np.float32)
        return O.select_keep(sc, np.arange(n), n, nk, S, W)
    if kind == "identity":
        return np.arange(nk)
    if kind == "hole_at_0":
        return np.arange(n - nk, n)
    if kind == "hole_at_end":
        return np.arange(nk)
    if kind == "every_other":
        return np.arange(0, n, 2)[:nk]
    if kind == "random":
        return np.sort(rng.choice(n, nk, replace=False))
    raise ValueError(kind)


COMPACT_CASES = [
    # dtype, head_dim, batch, H, len, n_keep, kind
    ("bf16", 128, 2, 8, 1152, 1024, "select"),
    ("bf16", 128, 1, 4, 2304, 2048, "random"),
    ("bf16", 128, 1, 2, 600, 300, "every_other"),
    ("bf16", 128, 1, 2, 600, 300, "hole_at_0"),
    ("bf16", 128, 1, 2, 600, 300, "hole_at_end"),
    ("bf16", 128, 1, 2, 600, 600, "identity"),
    ("f32", 64, 1, 2, 193, 192, "select"),
    ("f32", 64, 1, 2, 512, 192, "select"),
    ("bf16", 64, 2, 3, 1000, 517, "random"),
    ("f32", 128, 1, 2, 900, 450, "random"),
    ("bf16", 128, 1, 8, 131072, 39321, "random"),
    # one workgroup per slice up to n_keep = 4096, the grouped kernel beyond
    ("bf16", 128, 4, 8, 8192, 1024, "random"),     # prompt compression
    ("bf16", 128, 1, 2, 9000, 4096, "random"),
    ("bf16", 128, 1, 2, 9000, 4097, "random"),
    ("f32", 128, 1, 2, 5000, 4000, "hole_at_0"),
]


@pytest.mark.parametrize("case", COMPACT_CASES,
                         ids=[f"{c[0]}-d{c[1]}-n{c[4]}-k{c[5]}-{c[6]}"
                              for c in COMPACT_CASES])
def test_compact_bit_exact(case):
    import torch
    k = kve()
    dt, D, B, H, n, nk, kind = case
    print(f"[compact] {case}", flush=True)
    cap = n + 3
    rng = np.random.default_rng(n + nk + D)
    shape = k.Shape(B, H, 1, D, cap, k.F32 if dt == "f32" else k.BF16)
    dev = torch.device("cuda")
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    K = torch.randn((B, H, cap, D), device=dev).to(tdt)
    V = torch.randn((B, H, cap, D), device=dev).to(tdt)
    sc = torch.randn((B, H, cap), device=dev)
    pos = torch.arange(cap, dtype=torch.int32, device=dev).repeat(B, H, 1) * 3
    keeps = np.stack([[_keep_lists(rng, n, nk, 4, 64, kind) for _ in range(H)]
                      for _ in range(B)]).astype(np.int32)
    K0, V0, s0, p0 = K.clone(), V.clone(), sc.clone(), pos.clone()
    cache = k.CacheTensors(K, V, sc, pos)
    keep_t = torch.from_numpy(keeps).to(dev)
    k.kve_compact(shape, cache, n, keep_t, nk)
    torch.cuda.synchronize()
    # expected placement: the oracle's hole filling
    srcs = np.stack([[O.compaction_sources(keeps[b, h]) for h in range(H)]
                     for b in range(B)])
    idx = torch.from_numpy(srcs.astype(np.int64)).to(dev)
    expK = torch.gather(K0, 2, idx[..., None].expand(B, H, nk, D))
    expV = torch.gather(V0, 2, idx[..., None].expand(B, H, nk, D))
    iv = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(K[:, :, :nk].view(iv), expK.view(iv))
    assert torch.equal(V[:, :, :nk].view(iv), expV.view(iv))
    assert torch.equal(sc[:, :, :nk], torch.gather(s0, 2, idx))
    assert torch.equal(pos[:, :, :nk], torch.gather(p0, 2, idx))
    # slots from n_keep on are left as they were
    assert torch.equal(K[:, :, nk:].view(iv), K0[:, :, nk:].view(iv))
    assert torch.equal(pos[:, :, nk:], p0[:, :, nk:])
