"""a3 select and a4 compact on seeded random shapes against the oracle,
bit-exact: slice lengths from 2 to 60000 (the register, LDS-key and global
selects and their slot-count boundaries; the one-workgroup and the grouped
compactions), few or many slices, every score pattern of the fixed tests,
positions in slot order or shuffled, with and without temporal decay and
stochastic noise."""
import numpy as np
import pytest

import synthetic as syn
import test_gpu_select_compact as fixed
from test_gpu_stochastic import run_select

pytestmark = pytest.mark.gpu

PATTERNS = ["normal", "ties3", "const", "zeros", "sigmoid", "wide"]


def _select_cases(n=32, seed=11):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        length = int(np.exp(rng.uniform(np.log(2.0), np.log(60000.0))))
        max_slices = max(1, min(300, 400000 // length))
        slices = int(np.exp(rng.uniform(0.0, np.log(max_slices + 1)))) or 1
        slices = max(1, min(slices, max_slices))
        H = int(rng.integers(1, min(8, slices) + 1))
        b = max(1, slices // H)
        S = int(rng.integers(0, 9))
        W = int(rng.integers(0, min(300, length // 2) + 1))
        if S + W >= length or rng.random() < 0.1:
            n_keep = length
            S, W = min(S, length), 0
        else:
            n_keep = int(rng.integers(S + W, length))
        out.append((b, H, length, n_keep, S, W,
                    PATTERNS[int(rng.integers(0, len(PATTERNS)))],
                    "shuffled" if rng.random() < 0.5 else "sorted",
                    bool(rng.random() < 0.3), bool(rng.random() < 0.3)))
    return out


SELECT_CASES = _select_cases()


@pytest.mark.parametrize("case", SELECT_CASES, ids=[
    f"b{c[0]}H{c[1]}n{c[2]}k{c[3]}S{c[4]}W{c[5]}-{c[6]}-{c[7]}"
    f"{'-decay' if c[8] else ''}{'-noise' if c[9] else ''}"
    for c in SELECT_CASES])
def test_random_select(case):
    b, H, length, n_keep, S, W, pattern, order, decay, noisy = case
    print(f"[random-select] {case}", flush=True)
    rng = np.random.default_rng(length * 7 + n_keep)
    scores = fixed._scores(rng, pattern, (b, H, length))
    if order == "sorted":
        pos = np.broadcast_to(np.arange(length), (b, H, length)).copy()
    else:
        pos = np.stack([[rng.permutation(length + 5)[:length] for _ in range(H)]
                        for _ in range(b)])
    lg = (np.log(np.linspace(0.9, 0.9999, H)).astype(np.float32)
          if decay else None)
    noise = syn.gumbel_noise(rng, (b, H, length)) if noisy else None
    got, ref = run_select(b, H, length + 3, length, n_keep, S, W, scores, pos,
                          noise, lg)
    np.testing.assert_array_equal(got, ref)


def _compact_cases(n=16, seed=12):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        length = int(np.exp(rng.uniform(np.log(2.0), np.log(20000.0))))
        nk = int(rng.integers(1, length + 1))
        kinds = ["random", "identity", "hole_at_0", "hole_at_end"]
        if nk >= 68 and nk < length:
            kinds.append("select")
        if nk <= (length + 1) // 2:
            kinds.append("every_other")
        kind = kinds[int(rng.integers(0, len(kinds)))]
        if kind == "identity":
            nk = length
        dt = "f32" if rng.random() < 0.3 else "bf16"
        out.append((dt, int(rng.choice([64, 128])), int(rng.integers(1, 3)),
                    int(rng.integers(1, 5)), length, nk, kind))
    return out


COMPACT_CASES = _compact_cases()


@pytest.mark.parametrize("case", COMPACT_CASES, ids=[
    f"{c[0]}-d{c[1]}-b{c[2]}H{c[3]}-n{c[4]}-k{c[5]}-{c[6]}"
    for c in COMPACT_CASES])
def test_random_compact(case):
    fixed.test_compact_bit_exact(case)
