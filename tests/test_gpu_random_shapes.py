"""kve_step end to end against the oracle's policy loop on seeded random
shapes and policies: batch, KV heads, group size (1..8), head_dim (64, 128),
bf16 or float32, sinks, window, k = B - S - W (down to 0), eviction length
(1..33), MLP width (16..200, multiples of 16 take the MFMA scorer, others
the VALU one), ReLU or SiLU, plain or structured rows. Each case runs past
at least two evictions; every step is checked as in the fixed-shape tests
(retained set, scores, attention, lse through the harness). Further cases
score with the hidden-state gate (input widths in multiples of 32, up to 16
KV heads), whose pending hidden states are buffered between evictions."""
import numpy as np
import pytest

import synthetic as syn
from test_gpu_step import run_e2e

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        S = int(rng.integers(0, 7))
        W = int(rng.integers(1, 65))
        k = int(rng.choice([0, int(rng.integers(1, 120))]))
        L = int(rng.choice([1, 2, 7, 16, 33]))
        B = S + W + k
        n0 = int(B + rng.integers(-min(B - 1, 40), 300))
        hidden = int(rng.choice([16, 32, 48, 64, 96, 128, 24, 200]))
        out.append(dict(
            batch=int(rng.integers(1, 4)), n_kv=int(rng.integers(1, 4)),
            group=int(rng.choice([1, 2, 3, 4, 5, 8])), head_dim=d,
            kv_dtype=dtype, n0=max(n0, 1), sinks=S, window=W, budget=B,
            evict_len=L,
            steps=max(0, B - n0) + 2 * L + int(rng.integers(3, 40)),
            hidden=hidden, act=str(rng.choice(["relu", "silu"])),
            structured=bool(rng.random() < 0.5), name=f"random-{i}"))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[
    f"b{c['batch']}h{c['n_kv']}g{c['group']}d{c['head_dim']}{c['kv_dtype']}"
    f"-S{c['sinks']}W{c['window']}B{c['budget']}L{c['evict_len']}"
    f"-hid{c['hidden']}{c['act']}" for c in CASES])
def test_random_shape_end_to_end(case):
    print(f"[random-shape] {case}", flush=True)
    w = syn.workload(2, layers=1, **case)
    evictions, _ = run_e2e(w, seed=3)
    assert evictions >= 2


def _gate_cases(n=10, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(0, 7))
        W = int(rng.integers(1, 65))
        k = int(rng.choice([0, int(rng.integers(1, 120))]))
        L = int(rng.choice([1, 2, 7, 16, 33, 64]))
        B = S + W + k
        n0 = int(B + rng.integers(-min(B - 1, 40), 300))
        out.append(dict(
            batch=int(rng.integers(1, 3)), n_kv=int(rng.choice([1, 2, 5, 8, 16])),
            group=int(rng.choice([1, 2, 4, 5, 8])),
            head_dim=int(rng.choice([64, 128])), kv_dtype="bf16",
            n0=max(n0, 1), sinks=S, window=W, budget=B, evict_len=L,
            steps=max(0, B - n0) + 2 * L + int(rng.integers(3, 30)),
            hidden=32 * int(rng.integers(1, 65)), structured=False,
            name=f"random-gate-{i}"))
    return out


GATE_CASES = _gate_cases()


@pytest.mark.parametrize("case", GATE_CASES, ids=[
    f"b{c['batch']}h{c['n_kv']}g{c['group']}d{c['head_dim']}"
    f"-S{c['sinks']}W{c['window']}B{c['budget']}L{c['evict_len']}"
    f"-D{c['hidden']}" for c in GATE_CASES])
def test_random_gate_end_to_end(case):
    print(f"[random-gate] {case}", flush=True)
    w = syn.workload(5, layers=1, **case)
    evictions, _ = run_e2e(w, seed=4)
    assert evictions >= 2


DECAY_CASES = _cases(n=8, seed=20261205)


@pytest.mark.parametrize("case", DECAY_CASES, ids=[
    f"b{c['batch']}h{c['n_kv']}g{c['group']}d{c['head_dim']}{c['kv_dtype']}"
    f"-S{c['sinks']}W{c['window']}B{c['budget']}L{c['evict_len']}"
    for c in DECAY_CASES])
def test_random_shape_end_to_end_with_decay(case):
    """The same loop with temporal decay in the ranking (one decay rate
    per KV head, from 0.9 to 1 - 1e-6)."""
    print(f"[random-decay] {case}", flush=True)
    w = syn.workload(2, layers=1, **case)
    gammas = np.linspace(0.9, 1 - 1e-6, w.n_kv)
    evictions, _ = run_e2e(w, seed=7, gammas=gammas)
    assert evictions >= 2
