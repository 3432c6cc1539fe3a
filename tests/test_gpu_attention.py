"""a5 decode attention: HIP kernel vs the float64 oracle, element by element.

Sizes span several workgroup passes (32 rows), several splits and ragged
tails; slots beyond len hold NaN so any read past the retained rows would
show. Tolerance: 2e-3 * max|out| (float32 accumulation over bf16 inputs).
"""
import zlib

import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import attn_close, kve, LSE_ATOL

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, head_dim, group, n_kv, batch, len, capacity, key scale
    ("f32", 64, 2, 2, 1, 192, 256, 1.0),        # tiny workload shape
    ("bf16", 128, 4, 8, 96, 1088, 1152, 1.0),   # batch-96 stack layer: no split
    ("bf16", 128, 4, 8, 96, 1025, 1152, 1.0),   # ragged tail, no split
    ("bf16", 128, 4, 8, 16, 1087, 1152, 1.0),   # batch-16 layer: split
    ("bf16", 128, 4, 8, 8, 2175, 2304, 1.0),    # batch-8, B=2048 layer
    ("bf16", 64, 2, 8, 64, 333, 400, 1.0),      # d = 64, many slices
    ("f32", 128, 4, 8, 48, 257, 260, 1.0),      # float32, many slices
    ("bf16", 128, 4, 8, 2, 1087, 1152, 1.0),    # Qwen3-4B layer, mid-cycle
    ("bf16", 128, 4, 8, 2, 1024, 1152, 1.0),    # right after an eviction
    ("bf16", 128, 4, 2, 1, 1, 64, 1.0),         # single retained row
    ("bf16", 128, 4, 2, 1, 33, 64, 1.0),        # ragged tail
    ("bf16", 128, 5, 8, 1, 5000, 5000, 1.0),    # group 5, many splits
    ("bf16", 128, 5, 8, 1, 39353, 39385, 1.0),  # Qwen2.5-14B decode layer
    ("bf16", 64, 1, 3, 2, 300, 320, 1.0),
    ("f32", 128, 8, 2, 1, 700, 700, 1.0),
    ("bf16", 128, 3, 4, 3, 4097, 4100, 1.0),
    ("bf16", 128, 4, 2, 2, 2000, 2048, 6.0),    # peaked softmax
    ("f32", 64, 2, 2, 1, 2303, 2304, 4.0),
    # float32 rows of 16 lanes with whole quads of heads: the reduce-scatter
    # path with q scaled at load (its logits were once scaled twice)
    ("f32", 64, 4, 2, 2, 300, 320, 1.0),
    ("f32", 64, 8, 3, 1, 8, 69, 1.0),
]


def _rows(rng, shape, dtype, scale):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return syn.Stored(x, dtype)


def _poison(t, length):
    import torch
    t[:, :, length:] = float("nan")


def _random_cases(n=24, seed=7):
    """Seeded random shapes: group 1..8, d 64 or 128, bf16 or float32,
    lengths from 1 to ~8000 (every split count the planner picks for them),
    at most ~150k retained rows in all."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        length = int(np.exp(rng.uniform(0.0, np.log(8000.0))))
        slices = int(rng.integers(1, max(2, min(96, 150000 // length))))
        H = int(rng.integers(1, min(8, slices) + 1))
        B = max(1, slices // H)
        out.append(("f32" if rng.random() < 0.3 else "bf16",
                    int(rng.choice([64, 128])), int(rng.integers(1, 9)), H, B,
                    length, length + int(rng.integers(0, 65)),
                    float(rng.choice([1.0, 3.0, 6.0]))))
    return out


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-g{c[2]}-b{c[4]}-n{c[5]}"
                                             for c in CASES])
def test_decode_attention_matches_oracle(case):
    _check(case)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[
    f"{c[0]}-d{c[1]}-g{c[2]}-h{c[3]}-b{c[4]}-n{c[5]}" for c in RANDOM_CASES])
def test_decode_attention_random_shapes(case):
    _check(case)


def _check(case):
    import torch
    k = kve()
    dt, D, G, H, B, n, cap, kscale = case
    print(f"[attn] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    Ks = _rows(rng, (B, H, cap, D), dt, kscale)
    Vs = _rows(rng, (B, H, cap, D), dt, 1.0)
    Qs = _rows(rng, (B, H * G, D), dt, 1.0)
    shape = k.Shape(B, H, G, D, cap, k.F32 if dt == "f32" else k.BF16)
    dev = torch.device("cuda")
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(Ks.torch(dev))
    cache.v.copy_(Vs.torch(dev))
    _poison(cache.k, n)
    _poison(cache.v, n)
    q = Qs.torch(dev)
    out = torch.full((B, H * G, D), float("nan"), device=dev)
    lse = torch.full((B, H * G), float("nan"), device=dev)
    ws = k.alloc_workspace(shape, n, dev)
    k.kve_decode_attn(shape, cache, n, q, out, lse, ws)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    got_lse = lse.cpu().double().numpy()
    for b in range(B):
        for h in range(H):
            ref, ref_lse = O.decode_attention(Qs.f64[b, h * G:(h + 1) * G],
                                              Ks.f64[b, h, :n],
                                              Vs.f64[b, h, :n])
            attn_close(got[b, h * G:(h + 1) * G], ref, f"b{b} h{h}")
            np.testing.assert_allclose(got_lse[b, h * G:(h + 1) * G], ref_lse,
                                       atol=LSE_ATOL, rtol=1e-5)


def test_decode_attention_deterministic_and_len_sweep():
    """Bitwise-identical reruns; every len from 1 to 130 on one shape."""
    import torch
    k = kve()
    rng = np.random.default_rng(5)
    B, H, G, D, cap = 1, 2, 4, 128, 160
    Ks = _rows(rng, (B, H, cap, D), "bf16", 1.0)
    Vs = _rows(rng, (B, H, cap, D), "bf16", 1.0)
    Qs = _rows(rng, (B, H * G, D), "bf16", 1.0)
    shape = k.Shape(B, H, G, D, cap, k.BF16)
    dev = torch.device("cuda")
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(Ks.torch(dev))
    cache.v.copy_(Vs.torch(dev))
    q = Qs.torch(dev)
    ws = k.alloc_workspace(shape, cap, dev)
    out = torch.empty((B, H * G, D), device=dev)
    for n in list(range(1, 131)) + [cap]:
        k.kve_decode_attn(shape, cache, n, q, out, None, ws)
        first = out.clone()
        k.kve_decode_attn(shape, cache, n, q, out, None, ws)
        assert torch.equal(first, out), f"nondeterministic at len {n}"
        got = out.cpu().double().numpy()
        for h in range(H):
            ref, _ = O.decode_attention(Qs.f64[0, h * G:(h + 1) * G],
                                        Ks.f64[0, h, :n], Vs.f64[0, h, :n])
            attn_close(got[0, h * G:(h + 1) * G], ref, f"len {n} h{h}")


@pytest.mark.parametrize("batch,n", [(96, 1088), (2, 1087)],
                         ids=["unsplit-b96", "split-b2"])
def test_decode_attention_in_hip_graph(batch, n):
    """The decode-attention launches (attention, and the split merge when
    the rows are split) replay from a captured HIP graph: the library
    allocates nothing and records no memset, so every replay, with eager
    launches and synchronisations between replays, equals the eager result
    bitwise and the oracle within tolerance."""
    import torch
    k = kve()
    B, H, G, D, cap = batch, 8, 4, 128, 1152
    print(f"[attn-graph] batch {B} len {n}", flush=True)
    rng = np.random.default_rng(B * 1000 + n)
    Ks = _rows(rng, (B, H, cap, D), "bf16", 1.0)
    Vs = _rows(rng, (B, H, cap, D), "bf16", 1.0)
    Qs = _rows(rng, (B, H * G, D), "bf16", 1.0)
    Q2 = _rows(rng, (B, H * G, D), "bf16", 1.0)
    shape = k.Shape(B, H, G, D, cap, k.BF16)
    dev = torch.device("cuda")
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(Ks.torch(dev))
    cache.v.copy_(Vs.torch(dev))
    q, q2 = Qs.torch(dev), Q2.torch(dev)
    out = torch.empty((B, H * G, D), device=dev)
    lse = torch.empty((B, H * G), device=dev)
    out2 = torch.empty_like(out)
    ws = k.alloc_workspace(shape, cap, dev)
    k.kve_decode_attn(shape, cache, n, q, out, lse, ws)
    torch.cuda.synchronize()
    eager, eager_lse = out.clone(), lse.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            k.kve_decode_attn(shape, cache, n, q, out, lse, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: output differs"
        assert torch.equal(lse, eager_lse), f"replay {rep}: lse differs"
        # eager work on the same workspace between replays
        k.kve_decode_attn(shape, cache, n, q2, out2, None, ws)
        torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    for b in range(0, B, max(1, B // 4)):
        for h in range(H):
            ref, _ = O.decode_attention(Qs.f64[b, h * G:(h + 1) * G],
                                        Ks.f64[b, h, :n], Vs.f64[b, h, :n])
            attn_close(got[b, h * G:(h + 1) * G], ref, f"b{b} h{h}")
