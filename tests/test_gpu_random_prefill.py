"""Prefill selection (ranks and cutoffs, bit-exact) and the Eq. 26 masked
prefill attention (within the attention contract) on seeded random shapes:
prompt lengths that end anywhere inside a 64-query block or a sort chunk,
group sizes 1..8 (one or two heads per workgroup), d 64 or 128, sinks,
windows and budgets from k = 0 to k beyond the prompt, with and without
temporal decay."""
import numpy as np
import pytest

import oracle as O
import test_gpu_prefill as fixed

pytestmark = pytest.mark.gpu


def _select_cases(n=16, seed=21):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        length = int(np.exp(rng.uniform(0.0, np.log(9000.0))))
        S = int(rng.integers(0, 9))
        W = int(rng.integers(0, 200))
        k = int(rng.choice([0, int(rng.integers(1, max(2, length)))]))
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), length,
                    S, W, k, "ties" if rng.random() < 0.4 else "normal",
                    bool(rng.random() < 0.4)))
    return out


def _attn_cases(n=12, seed=22):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        length = int(np.exp(rng.uniform(0.0, np.log(520.0))))
        S = int(rng.integers(0, 6))
        W = int(rng.integers(1, 80))
        k = int(rng.choice([0, int(rng.integers(1, 300))]))
        out.append((1, int(rng.integers(1, 3)), int(rng.integers(1, 9)),
                    int(rng.choice([64, 128])), length, S, W, k,
                    bool(rng.random() < 0.4)))
    return out


SELECT_CASES = _select_cases()
ATTN_CASES = _attn_cases()


@pytest.mark.parametrize("case", SELECT_CASES, ids=[
    f"b{c[0]}H{c[1]}n{c[2]}S{c[3]}W{c[4]}k{c[5]}-{c[6]}{'-decay' if c[7] else ''}"
    for c in SELECT_CASES])
def test_random_prefill_select(case):
    b, H, n, S, W, k, kind, decay = case
    print(f"[random-prefill-select] {case}", flush=True)
    s, lg, rank, tau, *_ = fixed.run_select(b, H, n, S, W, k, kind, decay,
                                            seed=n * 3 + k)
    for bi in range(b):
        for h in range(H):
            r = O.prefill_ranks(s[bi, h], None if lg is None else float(lg[h]))
            assert np.array_equal(rank[bi, h], r), (bi, h)
            assert np.array_equal(tau[bi, h], O.prefill_cutoffs(r, S, W, k)), (bi, h)


@pytest.mark.parametrize("case", ATTN_CASES, ids=[
    f"H{c[1]}G{c[2]}d{c[3]}n{c[4]}S{c[5]}W{c[6]}k{c[7]}{'-decay' if c[8] else ''}"
    for c in ATTN_CASES])
def test_random_prefill_attention(case):
    b, H, G, d, n, S, W, k, decay = case
    print(f"[random-prefill-attn] {case}", flush=True)
    rank, tau, K, V, Q, out, lse = fixed.run_attn(b, H, G, d, n, S, W, k,
                                                  seed=n * 5 + k, decay=decay)
    for bi in range(b):
        masks = np.stack([O.prefill_mask(rank[bi, h], tau[bi, h], S, W)
                          for h in range(H)])
        ref, ref_lse = O.prefill_attention(Q.f64[bi], K.f64[bi], V.f64[bi],
                                           masks, G)
        fixed.assert_attention_close(out[bi], ref, f"batch {bi}")
        np.testing.assert_allclose(lse[bi], ref_lse, rtol=0,
                                   atol=fixed.LSE_TOL)
