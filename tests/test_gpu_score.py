"""a2 scorers: MFMA / VALU MLP over [k; v] and the MFMA hidden-state gate,
against the float64 oracle, within 1e-3 absolute."""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import kve, SCORE_ATOL

pytestmark = pytest.mark.gpu

MLP_CASES = [
    # dtype, head_dim, hidden, act, batch, H, rows (slot range), cap
    ("bf16", 128, 64, "relu", 16, 8, (1024, 1152), 1152),   # Qwen3-4B, L=128
    ("bf16", 128, 64, "relu", 1, 8, (0, 8192), 8192),       # prefill
    # workgroup sizing by row count (256 CUs): a batch-96 decode eviction
    # (2 tiles per wave), a prompt long enough for 8 tiles per wave
    ("bf16", 128, 64, "relu", 96, 8, (1024, 1152), 1152),
    ("bf16", 128, 64, "relu", 8, 8, (0, 8192), 8192),
    ("bf16", 128, 64, "silu", 2, 3, (5, 77), 100),
    ("bf16", 128, 32, "relu", 2, 2, (0, 33), 40),
    ("bf16", 64, 48, "relu", 1, 2, (3, 200), 256),
    ("bf16", 128, 40, "relu", 1, 2, (0, 100), 100),          # VALU bf16 path
    ("f32", 64, 32, "relu", 1, 2, (0, 512), 512),            # tiny workload
    ("f32", 64, 32, "silu", 1, 2, (192, 193), 193),
    ("f32", 128, 20, "relu", 2, 2, (0, 70), 70),
]


@pytest.mark.parametrize("case", MLP_CASES,
                         ids=[f"{c[0]}-d{c[1]}-h{c[2]}-{c[3]}-r{c[6][1]-c[6][0]}"
                              for c in MLP_CASES])
def test_mlp_scores(case):
    import torch
    k = kve()
    dt, D, hid, act, B, H, (r0, r1), cap = case
    print(f"[score] {case}", flush=True)
    rng = np.random.default_rng(D * 1000 + hid + r1)
    Ks = syn.Stored((rng.standard_normal((B, H, cap, D)) * 1.5).astype(
        np.float32), dt)
    Vs = syn.Stored(rng.standard_normal((B, H, cap, D)).astype(np.float32), dt)
    w1 = syn.Stored((rng.standard_normal((H, hid, 2 * D)) / np.sqrt(2 * D)
                     ).astype(np.float32), dt)
    w2 = syn.Stored((rng.standard_normal((H, hid)) / np.sqrt(hid)).astype(
        np.float32), "f32")
    b1 = syn.Stored((0.1 * rng.standard_normal((H, hid))).astype(np.float32),
                    "f32")
    b2 = syn.Stored((0.1 * rng.standard_normal(H)).astype(np.float32), "f32")
    shape = k.Shape(B, H, 1, D, cap, k.F32 if dt == "f32" else k.BF16)
    dev = torch.device("cuda")
    cache = k.CacheTensors.empty(shape, dev)
    cache.k.copy_(Ks.torch(dev))
    cache.v.copy_(Vs.torch(dev))
    cache.score.fill_(12345.0)
    sc = k.Scorer.mlp(w1.torch(dev), w2.torch(dev), b1.torch(dev),
                      b2.torch(dev), act=k.ACT_RELU if act == "relu"
                      else k.ACT_SILU)
    k.kve_score(shape, sc, cache, r0, r1)
    got = cache.score.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = O.mlp_score(Ks.f64[b, h, r0:r1], Vs.f64[b, h, r0:r1],
                              w1.f64[h], b1.f64[h], w2.f64[h], b2.f64[h], act)
            np.testing.assert_allclose(got[b, h, r0:r1], ref, rtol=0,
                                       atol=SCORE_ATOL)
            # slots outside the range are untouched
            assert np.all(got[b, h, :r0] == 12345.0)
            assert np.all(got[b, h, r1:] == 12345.0)


GATE_CASES = [
    # batch, H, D, rows, slot_begin, cap
    (1, 8, 5120, 300, 0, 300),      # Qwen2.5-14B hidden size
    (1, 8, 5120, 64, 39321, 39385),  # a decode buffer of L = 64 tokens
    (2, 3, 256, 77, 10, 100),
    (1, 16, 1024, 130, 0, 130),
    # at most 64 rows: the contraction split over 16 waves
    (3, 16, 32, 1, 5, 10),           # one k step, one row
    (2, 5, 1056, 50, 3, 60),         # 33 k steps: 3 per wave, no full block
    (1, 8, 5120, 63, 0, 64),         # ragged group
    (2, 8, 8192, 64, 0, 64),         # 16 k steps per wave: four full blocks
]


@pytest.mark.parametrize("case", GATE_CASES,
                         ids=[f"b{c[0]}H{c[1]}D{c[2]}r{c[3]}" for c in GATE_CASES])
def test_gate_scores(case):
    import torch
    k = kve()
    B, H, Dh, rows, s0, cap = case
    print(f"[gate] {case}", flush=True)
    rng = np.random.default_rng(Dh + rows)
    hid = syn.Stored(rng.standard_normal((B, rows, Dh)).astype(np.float32),
                     "bf16")
    gw = syn.Stored((rng.standard_normal((H, Dh)) / np.sqrt(Dh)).astype(
        np.float32), "bf16")
    gb = syn.Stored((0.3 * rng.standard_normal(H)).astype(np.float32), "f32")
    shape = k.Shape(B, H, 5, 128, cap, k.BF16)
    dev = torch.device("cuda")
    tiny = torch.zeros(1, device=dev)
    score = torch.full((B, H, cap), -7.0, device=dev)
    cache = k.CacheTensors(tiny, tiny, score,
                           torch.zeros(1, dtype=torch.int32, device=dev))
    sc = k.Scorer.gate(gw.torch(dev), gb.torch(dev))
    k.kve_score(shape, sc, cache, s0, s0 + rows, hidden=hid.torch(dev))
    got = score.cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = O.gate_score(hid.f64[b], gw.f64[h], gb.f64[h])
            np.testing.assert_allclose(got[b, h, s0:s0 + rows], ref, rtol=0,
                                       atol=SCORE_ATOL)
            assert np.all(got[b, h, :s0] == -7.0)
            assert np.all(got[b, h, s0 + rows:] == -7.0)
