"""The low-rank sink-attention gate and the stateful mLSTM scorer on seeded
random shapes against the float64 oracle, each at its fixed tests'
tolerance: the gate over input widths in multiples of 32, groups 1..8,
0..16 sink keys, one row to several hundred at any slot offset; the mLSTM
at head_dim 64 or 128 with read-out delays from 0 past the prompt length
and the absorption split over up to five calls at random cuts (older rows
shuffled between calls, as compaction moves them). Both also run through
kve_step end to end on seeded random shapes and policies against the
oracle's policy loop."""
import numpy as np
import pytest

import synthetic as syn
import test_gpu_mlstm as fixed_mlstm
import test_gpu_sink_gate as fixed_gate

pytestmark = pytest.mark.gpu


def _gate_cases(n=12, seed=41):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = 32 * int(rng.integers(1, 161))
        rows = int(np.exp(rng.uniform(0.0, np.log(700.0))))
        s0 = int(rng.integers(0, 64))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 9)),
                    int(rng.integers(1, 9)), D, rows, s0,
                    s0 + rows + int(rng.integers(0, 5)),
                    int(rng.integers(0, 17))))
    return out


def _mlstm_cases(n=10, seed=42):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        b, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        tokens = int(rng.integers(1, 700))
        W = int(rng.choice([0, 1, 16, 64, 128, 200, 800]))
        calls = int(rng.integers(1, 6))
        cuts = sorted(set(int(c) for c in rng.integers(1, tokens + 1, calls - 1)))
        out.append((b, H, d, tokens, W, tuple(cuts + [tokens]) if
                    (not cuts or cuts[-1] != tokens) else tuple(cuts)))
    return out


GATE_CASES = _gate_cases()
MLSTM_CASES = _mlstm_cases()


@pytest.mark.parametrize("case", GATE_CASES, ids=[
    f"b{c[0]}H{c[1]}G{c[2]}D{c[3]}r{c[4]}s{c[5]}S{c[7]}" for c in GATE_CASES])
def test_random_sink_gate_scores(case):
    fixed_gate.test_sink_gate_scores(case)


@pytest.mark.parametrize("case", MLSTM_CASES, ids=[
    f"b{c[0]}H{c[1]}d{c[2]}n{c[3]}W{c[4]}calls{len(c[5])}"
    for c in MLSTM_CASES])
def test_random_mlstm_scores(case):
    print(f"[mlstm-random] {case}", flush=True)
    fixed_mlstm.run_case(*case, seed=1000 + sum(case[:5]))


def _step_cases(scorer, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(0, 7))
        W = int(rng.integers(1, 65))
        k = int(rng.choice([0, int(rng.integers(1, 100))]))
        L = int(rng.choice([1, 2, 7, 16, 33]))
        B = S + W + k
        n0 = int(B + rng.integers(-min(B - 1, 30), 200))
        d = int(rng.choice([64, 128]))
        c = dict(batch=int(rng.integers(1, 3)), n_kv=int(rng.integers(1, 4)),
                 group=int(rng.choice([1, 2, 4, 5, 8])), head_dim=d,
                 kv_dtype="bf16", sinks=S, window=W, budget=B, evict_len=L,
                 structured=False, name=f"random-{scorer}-{i}")
        if scorer == "mlstm":
            # the read-out delay is the window: the prompt holds at least W
            c.update(n0=max(n0, W + 1), hidden=d // 2, scorer="mlstm")
        else:
            c.update(n0=max(n0, 1), hidden=32 * int(rng.integers(1, 41)),
                     scorer="sink_gate")
        c["steps"] = max(0, B - c["n0"]) + 2 * L + int(rng.integers(3, 25))
        out.append(c)
    return out


SG_STEP_CASES = _step_cases("sink_gate", 8, 43)
MLSTM_STEP_CASES = _step_cases("mlstm", 8, 44)


def _step_id(c):
    return (f"b{c['batch']}h{c['n_kv']}g{c['group']}d{c['head_dim']}"
            f"-S{c['sinks']}W{c['window']}B{c['budget']}L{c['evict_len']}"
            f"-n{c['n0']}-hid{c['hidden']}")


@pytest.mark.parametrize("case", SG_STEP_CASES,
                         ids=[_step_id(c) for c in SG_STEP_CASES])
def test_random_sink_gate_step_end_to_end(case):
    """kve_step with the sink gate (buffered hidden states) on seeded random
    shapes and policies, past at least two evictions."""
    print(f"[sink-gate-step-random] {case}", flush=True)
    w = syn.workload(5, layers=1, **case)
    assert fixed_gate.run_e2e_sink_gate(w, seed=5, check_stride=1) >= 2


@pytest.mark.parametrize("case", MLSTM_STEP_CASES,
                         ids=[_step_id(c) for c in MLSTM_STEP_CASES])
def test_random_mlstm_step_end_to_end(case):
    """kve_step with the stateful scorer (read-out delayed by the window) on
    seeded random shapes and policies, past at least two evictions."""
    print(f"[mlstm-step-random] {case}", flush=True)
    w = syn.workload(2, layers=1, **case)
    assert fixed_mlstm.run_e2e_mlstm(w, seed=6) >= 2
