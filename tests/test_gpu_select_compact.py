"""a3 select and a4 compact: bit-exact against the oracle when both sides
are given the same float32 scores and positions, including every kind of
tie and caches whose slot order is not position order."""
import zlib

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
    (4, 64, 4096, 1024, 32, 8),    # 256 slices, keys in registers (limit)
    (4, 64, 4097, 1024, 4, 8),     # just past it: keys in LDS
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


FUSED_CASES = [
    # dtype, d, G, batch, H, B, L, S, W
    ("bf16", 128, 4, 12, 8, 1024, 128, 4, 128),   # batch-96 decode eviction
    ("bf16", 128, 4, 2, 8, 2048, 256, 4, 256),    # batch-8, B = 2048
    ("f32", 64, 2, 1, 2, 192, 1, 4, 64),          # tiny workload, L = 1
    ("bf16", 64, 2, 3, 4, 2048, 2048, 4, 2000),   # 4096 entries, 2048 moves
    ("bf16", 64, 2, 1, 4, 2049, 2048, 4, 2000),   # 4097: two launches
    ("bf16", 128, 1, 2, 3, 50, 20, 0, 0),         # nothing protected
    ("bf16", 64, 2, 4, 2, 300, 100, 4, 100),      # d = 64
]


@pytest.mark.parametrize("pending", ["one", "L"])
@pytest.mark.parametrize("mode", ["plain", "decay", "stochastic"])
@pytest.mark.parametrize("order", ["sorted", "shuffled"])
@pytest.mark.parametrize("pattern", ["normal", "ties3", "zeros"])
@pytest.mark.parametrize("case", FUSED_CASES, ids=[
    f"{c[0]}d{c[1]}b{c[3]}B{c[5]}L{c[6]}" for c in FUSED_CASES])
def test_step_eviction_equals_separate_calls(case, pattern, order, mode,
                                             pending):
    """An evicting kve_step selects and compacts in one launch when the
    slice is short (the kept list stays on chip), and with a bf16 MLP scorer
    and up to 128 pending rows (pending "L": the L newest rows unscored, as
    at a periodic eviction) it also appends and scores them in that launch.
    Either way it must leave exactly the cache and kept slots that
    kve_append, kve_score, kve_select_evict and kve_compact leave, bitwise,
    whatever the ties, decay or noise."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    dt, D, G, batch, H, B, L, S, W = case
    print(f"[fused-evict] {case} {pattern} {order} {mode} {pending}",
          flush=True)
    rng = np.random.default_rng(zlib.crc32(repr((case, pattern, order, mode,
                                                 pending)).encode()))
    cap = B + L
    n = cap - 1  # the next step appends at slot n and evicts
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    shape = k.Shape(batch, H, G, D, cap, k.F32 if dt == "f32" else k.BF16)
    sc_np = np.zeros((batch, H, cap), np.float32)
    sc_np[:, :, :n] = _scores(rng, pattern, (batch, H, n))
    pos_np = _positions(rng, batch, H, cap, n, order)
    kv = [torch.from_numpy(rng.standard_normal((batch, H, cap, D))
                           .astype(np.float32)).to(tdt) for _ in range(2)]
    lg = gum = None
    if mode == "decay":
        lg = torch.from_numpy(np.log(rng.uniform(0.9, 0.999999, H))
                              .astype(np.float32)).to(dev)
    if mode == "stochastic":
        u = rng.uniform(1e-7, 1 - 1e-7, (batch, H, cap))
        gum = torch.from_numpy(-np.log(-np.log(u)).astype(np.float32)).to(dev)
    pol = k.Policy(B, S, W, L, log_gamma=lg, gumbel=gum)
    caches = []
    for _ in range(2):
        c = k.CacheTensors.empty(shape, dev)
        c.k.copy_(kv[0])
        c.v.copy_(kv[1])
        c.score.copy_(torch.from_numpy(sc_np))
        c.pos.copy_(torch.from_numpy(pos_np.astype(np.int32)))
        caches.append(c)
    w1 = torch.from_numpy((rng.standard_normal((H, 16, 2 * D)) *
                           (2 * D) ** -0.5).astype(np.float32)).to(tdt).to(dev)
    w2 = torch.from_numpy(rng.standard_normal((H, 16)).astype(np.float32)
                          ).to(dev)
    scorer = k.Scorer.mlp(w1, w2)
    kn, vn, q = (torch.from_numpy(rng.standard_normal(sh).astype(np.float32))
                 .to(tdt).to(dev)
                 for sh in ((batch, H, D), (batch, H, D), (batch, H * G, D)))
    keeps = [torch.full((batch, H, B), -7, dtype=torch.int32, device=dev)
             for _ in range(2)]
    # fused: one evicting kve_step (nothing pending before it)
    out = torch.empty((batch, H * G, D), device=dev)
    ws = k.alloc_workspace(shape, cap, dev)
    pend0 = n if pending == "one" else B  # first unscored slot
    st = k.DecodeState(n, pend0, n)
    k.kve_step(shape, pol, scorer, caches[0], st, kn, vn, q, out, None,
               keeps[0], ws)
    assert st.evicted == 1 and st.len == B
    # separate calls on the other copy
    c = caches[1]
    k.kve_append(shape, c, n, n, kn, vn)
    k.kve_score(shape, scorer, c, pend0, n + 1)
    torch.cuda.synchronize()
    sc_all = c.score.cpu().numpy().copy()   # the appended rows' scores too
    k.kve_select_evict(shape, pol, c, n + 1, B, keeps[1])
    k.kve_compact(shape, c, n + 1, keeps[1], B)
    torch.cuda.synchronize()
    assert torch.equal(keeps[0], keeps[1])
    for name in ("k", "v", "score", "pos"):
        a, b = getattr(caches[0], name), getattr(caches[1], name)
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), name
    # the kept slots against the oracle's rule, and the compacted positions
    # slot by slot against its placement rule
    got_keep = keeps[0].cpu().numpy()
    got_pos = caches[0].pos.cpu().numpy()
    lgn = None if lg is None else lg.cpu().numpy()
    gn = None if gum is None else gum.cpu().numpy()
    pos_all = pos_np.copy()
    pos_all[:, :, n] = n
    for sl in range(min(batch * H, 16)):  # the separate calls cover all
        bi, h = divmod(sl, H)
        lgh = None if lgn is None else float(lgn[h])
        if gn is None:
            ref = O.select_keep(sc_all[bi, h, :n + 1], pos_all[bi, h, :n + 1],
                                n + 1, B, S, W, lgh)
        else:
            ref = O.select_keep_stochastic(
                sc_all[bi, h, :n + 1], pos_all[bi, h, :n + 1], n + 1, B, S,
                W, gn[bi, h, :n + 1], lgh)
        np.testing.assert_array_equal(got_keep[bi, h], ref,
                                      err_msg=f"slice {bi},{h}")
        src = O.compaction_sources(ref)
        np.testing.assert_array_equal(got_pos[bi, h, :B],
                                      pos_all[bi, h, src],
                                      err_msg=f"slice {bi},{h}")
