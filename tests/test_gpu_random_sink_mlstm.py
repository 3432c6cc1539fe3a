"""The low-rank sink-attention gate and the stateful mLSTM scorer on seeded
random shapes against the float64 oracle, each at its fixed tests'
tolerance: the gate over input widths in multiples of 32, groups 1..8,
0..16 sink keys, one row to several hundred at any slot offset; the mLSTM
at head_dim 64 or 128 with read-out delays from 0 past the prompt length
and the absorption split over up to five calls at random cuts (older rows
shuffled between calls, as compaction moves them)."""
import numpy as np
import pytest

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
