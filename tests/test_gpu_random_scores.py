"""a2 scorers on seeded random shapes against the float64 oracle (within
1e-3 absolute, slots outside the range untouched): the MLP over [k; v]
(head_dim 64 or 128, hidden widths that take the MFMA tiles and widths that
take the VALU kernel, bf16 or float32, ReLU or SiLU, row ranges from one row
to several thousand at any offset) and the hidden-state gate (input widths
in multiples of 32, from one row to a few hundred)."""
import numpy as np
import pytest

import test_gpu_score as fixed

pytestmark = pytest.mark.gpu


def _mlp_cases(n=20, seed=31):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        dt = "f32" if rng.random() < 0.3 else "bf16"
        hid = int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128, 8, 40, 200, 256]))
        rows = int(np.exp(rng.uniform(0.0, np.log(6000.0))))
        r0 = int(rng.integers(0, 200))
        slices_max = max(1, 60000 // rows)
        H = int(rng.integers(1, min(8, slices_max) + 1))
        B = int(rng.integers(1, max(2, min(32, slices_max // H) + 1)))
        out.append((dt, d, hid, str(rng.choice(["relu", "silu"])), B, H,
                    (r0, r0 + rows), r0 + rows + int(rng.integers(0, 9))))
    return out


def _gate_cases(n=12, seed=32):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D = 32 * int(rng.integers(1, 161))
        rows = int(np.exp(rng.uniform(0.0, np.log(400.0))))
        s0 = int(rng.integers(0, 50))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 17)), D, rows,
                    s0, s0 + rows + int(rng.integers(0, 5))))
    return out


MLP_CASES = _mlp_cases()
GATE_CASES = _gate_cases()


@pytest.mark.parametrize("case", MLP_CASES, ids=[
    f"{c[0]}-d{c[1]}-h{c[2]}-{c[3]}-b{c[4]}H{c[5]}-r{c[6][0]}:{c[6][1]}"
    for c in MLP_CASES])
def test_random_mlp_scores(case):
    fixed.test_mlp_scores(case)


@pytest.mark.parametrize("case", GATE_CASES, ids=[
    f"b{c[0]}H{c[1]}D{c[2]}r{c[3]}s{c[4]}" for c in GATE_CASES])
def test_random_gate_scores(case):
    fixed.test_gate_scores(case)
