"""Prefill selection and masked prefill attention (KVpop section 3.2
"Running top-k sparse attention", Appendix C.1-C.2, Eq. 26) through the C
ABI, against the float64 oracle.

Ranks and cutoffs are integers decided from the same float32 keys on both
sides: bit-exact. Attention is held to the attention contract: within
2e-3 * max|out| of the float64 oracle per (batch, query head) output tensor.
The GPU feeds each softmax weight to the P.V contraction as a float16
(relative error at most 2^-11) when every V element of the slice converts
to float16 (largest |v| in [2^-6, 65280]), else as two bf16 parts (its
rounding and the remainder, relative error at most 2^-17 together); it
normalises by the float32 sum. lse is float32 math on unrounded weights:
within 1e-4 absolute.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as syn
from kvharness import kve

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4
ATTN_RTOL = 2e-3   # |gpu - oracle| <= 2e-3 * max|out| per output tensor


def assert_attention_close(got, ref, what=""):
    """got, ref [H*G][n][d] of one batch row: each query head's output
    tensor within ATTN_RTOL of its largest oracle element."""
    for j in range(ref.shape[0]):
        tol = ATTN_RTOL * np.abs(ref[j]).max()
        err = np.abs(got[j] - ref[j]).max()
        assert err <= tol, f"{what} head {j}: |err| {err:.3g} > {tol:.3g}"


def scores_for(rng, b, H, n, kind):
    if kind == "ties":
        s = rng.integers(0, 5, (b, H, n)).astype(np.float32)
        s[..., ::11] = -0.0
        return s
    return rng.standard_normal((b, H, n)).astype(np.float32)


def run_select(b, H, n, S, W, k, kind, decay, seed, cap=None):
    import torch
    k_ = kve()
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed)
    cap = cap or n
    shape = k_.Shape(b, H, 1, 64, cap, k_.BF16)
    cache = k_.CacheTensors.empty(shape, dev)
    s = scores_for(rng, b, H, n, kind)
    cache.score[:, :, :n] = torch.from_numpy(s).to(dev)
    cache.score[:, :, n:] = float("nan")  # beyond the prompt: never read
    lg = None
    if decay:
        lg = np.log(np.linspace(0.9, 0.999999, H)).astype(np.float32)
    pol = k_.Policy(S + W + k, S, W, 1,
                    log_gamma=None if lg is None else torch.from_numpy(lg).to(dev))
    rank = torch.full((b, H, n), -7, dtype=torch.int32, device=dev)
    tau = torch.full((b, H, n), -7, dtype=torch.int32, device=dev)
    k_.kve_prefill_select(shape, pol, cache, n, rank, tau)
    torch.cuda.synchronize()
    return s, lg, rank.cpu().numpy(), tau.cpu().numpy(), cache, shape, pol


SELECT_CASES = [
    # b, H, n, S, W, k, scores, decay
    (1, 2, 1, 4, 8, 16, "normal", False),
    (2, 3, 7, 1, 2, 2, "ties", False),
    (1, 2, 300, 4, 16, 40, "ties", False),
    (2, 2, 300, 4, 16, 40, "normal", True),
    (1, 2, 4113, 4, 64, 500, "normal", False),   # two sort chunks, ragged
    (1, 1, 2000, 0, 0, 100, "ties", False),
    (1, 2, 500, 3, 5, 0, "normal", False),         # k = 0
    (1, 2, 500, 3, 5, 600, "normal", False),       # k > n: nothing cut
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=[
    f"b{c[0]}H{c[1]}n{c[2]}S{c[3]}W{c[4]}k{c[5]}-{c[6]}{'-decay' if c[7] else ''}"
    for c in SELECT_CASES])
def test_prefill_select_exact(case):
    b, H, n, S, W, k, kind, decay = case
    print(f"[prefill-select] {case}", flush=True)
    s, lg, rank, tau, *_ = run_select(b, H, n, S, W, k, kind, decay,
                                      seed=n + S + W + k)
    for bi in range(b):
        for h in range(H):
            r = O.prefill_ranks(s[bi, h], None if lg is None else float(lg[h]))
            assert np.array_equal(rank[bi, h], r), (bi, h)
            t = O.prefill_cutoffs(r, S, W, k)
            assert np.array_equal(tau[bi, h], t), (bi, h)


def test_prefill_last_row_is_one_shot_compression():
    """The mask row of the last prompt position keeps what the one-shot
    compression (kve_select_evict down to B) keeps."""
    import torch
    k_ = kve()
    b, H, n, S, W, k = 2, 4, 3000, 4, 128, 700
    s, lg, rank, tau, cache, shape, pol = run_select(b, H, n, S, W, k,
                                                     "ties", True, seed=9)
    cache.pos[:, :, :n] = torch.arange(n, dtype=torch.int32, device="cuda")
    keep = torch.zeros((b, H, S + W + k), dtype=torch.int32, device="cuda")
    k_.kve_select_evict(shape, pol, cache, n, S + W + k, keep)
    kept = keep.cpu().numpy()
    for bi in range(b):
        for h in range(H):
            M = O.prefill_mask(rank[bi, h], tau[bi, h], S, W)
            assert np.flatnonzero(M[n - 1]).tolist() == kept[bi, h].tolist()


ATTN_CASES = [
    # b, H, G, d, n, S, W, k
    (1, 2, 4, 128, 200, 4, 16, 40),
    (2, 1, 1, 128, 45, 2, 3, 10),
    (1, 2, 5, 128, 333, 4, 32, 64),      # G = 5: two head pairs, then the
                                         #   fifth head in a launch of its own
    (2, 2, 3, 64, 201, 3, 24, 50),       # G = 3, d = 64: a pair and one head
    (1, 2, 2, 64, 257, 1, 8, 100),
    (1, 1, 8, 128, 130, 0, 1, 20),
    (1, 2, 4, 128, 100, 4, 16, 200),     # k >= n: causal attention
    (1, 1, 3, 128, 1, 4, 8, 16),         # one token
    (1, 2, 4, 128, 150, 2, 0, 30),       # W = 0: no window, a query keeps
    (1, 1, 2, 64, 100, 0, 0, 10),        #   itself only among its top k
]


def run_attn(b, H, G, d, n, S, W, k, seed, decay=False, vscale=None):
    import torch
    k_ = kve()
    dev = torch.device("cuda")
    s, lg, rank, tau, cache, shape, pol = run_select(b, H, n, S, W, k, "normal",
                                                     decay, seed)
    shape = k_.Shape(b, H, G, d, n, k_.BF16)
    cache2 = k_.CacheTensors.empty(shape, dev)
    rng = np.random.default_rng(seed + 1)
    K = syn.Stored(rng.standard_normal((b, H, n, d)).astype(np.float32), "bf16")
    Vf = rng.standard_normal((b, H, n, d)).astype(np.float32)
    if vscale is not None:
        Vf *= np.asarray(vscale, np.float32)[None, :, None, None]
    V = syn.Stored(Vf, "bf16")
    Q = syn.Stored((1.5 * rng.standard_normal((b, H * G, n, d))).astype(np.float32),
                   "bf16")
    cache2.k.copy_(K.torch(dev))
    cache2.v.copy_(V.torch(dev))
    out = torch.full((b, H * G, n, d), float("nan"), device=dev)
    lse = torch.full((b, H * G, n), float("nan"), device=dev)
    k_.kve_prefill_attn(shape, pol, cache2, n,
                        torch.from_numpy(rank).to(dev),
                        torch.from_numpy(tau).to(dev), Q.torch(dev), out, lse)
    torch.cuda.synchronize()
    return rank, tau, K, V, Q, out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", ATTN_CASES, ids=[
    f"b{c[0]}H{c[1]}G{c[2]}d{c[3]}n{c[4]}S{c[5]}W{c[6]}k{c[7]}"
    for c in ATTN_CASES])
def test_prefill_attention(case):
    b, H, G, d, n, S, W, k = case
    print(f"[prefill-attn] {case}", flush=True)
    rank, tau, K, V, Q, out, lse = run_attn(*case, seed=sum(case))
    for bi in range(b):
        masks = np.stack([O.prefill_mask(rank[bi, h], tau[bi, h], S, W)
                          for h in range(H)])
        ref, ref_lse = O.prefill_attention(Q.f64[bi], K.f64[bi], V.f64[bi],
                                           masks, G)
        rel = max(np.abs(out[bi, j] - ref[j]).max() / np.abs(ref[j]).max()
                  for j in range(ref.shape[0]))
        print(f"[prefill-attn] max |err| / max|out| {rel:.3g}", flush=True)
        assert_attention_close(out[bi], ref, f"batch {bi}")
        np.testing.assert_allclose(lse[bi], ref_lse, rtol=0, atol=LSE_TOL)


VSCALE_CASES = [
    # b, H, G, d, n, S, W, k, V scale per KV head. N(0,1) rows of V times
    # the scale: 8e3 (largest |v| near 3e4, the float16 path near its top),
    # 1e5 (beyond 65280: bf16 weight pairs for that slice only), 0.01 (the
    # float16 path with values among float16's subnormals), 1e-7 (largest
    # |v| below 2^-6: bf16 weight pairs)
    (1, 2, 4, 128, 300, 4, 16, 60, (1.0, 8e3)),
    (1, 2, 4, 128, 300, 4, 16, 60, (1.0, 1e5)),
    (1, 2, 4, 128, 300, 4, 16, 60, (0.01, 1e-7)),
    (1, 2, 2, 64, 257, 1, 8, 100, (1e5, 1.0)),
]


@pytest.mark.parametrize("case", VSCALE_CASES, ids=[
    f"d{c[3]}-v{c[8][0]:g},{c[8][1]:g}" for c in VSCALE_CASES])
def test_prefill_attention_v_range(case):
    """Slices whose V leaves float16's range take the bf16 path, the others
    the float16 one; both within the contract."""
    b, H, G, d, n, S, W, k, vs = case
    print(f"[prefill-attn-vrange] {case}", flush=True)
    rank, tau, K, V, Q, out, lse = run_attn(b, H, G, d, n, S, W, k,
                                            seed=n + d, vscale=vs)
    masks = np.stack([O.prefill_mask(rank[0, h], tau[0, h], S, W)
                      for h in range(H)])
    ref, ref_lse = O.prefill_attention(Q.f64[0], K.f64[0], V.f64[0], masks, G)
    rel = max(np.abs(out[0, j] - ref[j]).max() / np.abs(ref[j]).max()
              for j in range(ref.shape[0]))
    print(f"[prefill-attn-vrange] max |err| / max|out| {rel:.3g}", flush=True)
    assert_attention_close(out[0], ref, f"{vs}")
    np.testing.assert_allclose(lse[0], ref_lse, rtol=0, atol=LSE_TOL)


def test_prefill_attention_with_decay_and_skipped_blocks():
    """Decay orders eligible tokens by age as well as score: whole key
    blocks fall below the cutoff and are skipped."""
    b, H, G, d, n, S, W, k = 1, 2, 4, 128, 1500, 4, 64, 96
    rank, tau, K, V, Q, out, lse = run_attn(b, H, G, d, n, S, W, k, seed=3,
                                            decay=True)
    masks = np.stack([O.prefill_mask(rank[0, h], tau[0, h], S, W)
                      for h in range(H)])
    ref, ref_lse = O.prefill_attention(Q.f64[0], K.f64[0], V.f64[0], masks, G)
    assert_attention_close(out[0], ref, "decay")
    np.testing.assert_allclose(lse[0], ref_lse, rtol=0, atol=LSE_TOL)


FULL_CASES = [
    # b, H, G, n, S, W, B: a Qwen3-4B layer (8192-token prompt, B = 1024)
    # and a Qwen2.5-14B layer (131072-token prompt, 30% budget)
    (2, 8, 4, 8192, 4, 128, 1024),
    (1, 8, 5, 131072, 4, 512, 39321),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=[f"n{c[3]}" for c in FULL_CASES])
def test_prefill_full_size_sampled(case):
    """Full-size prompts in the launch shape the benchmark uses: ranks exact
    for every token, cutoffs exact at sampled positions (the definition:
    sort of the eligible ranks), attention rows at sampled (position, head)
    pairs against decode attention over the tokens the mask keeps. The
    sampled rows always include position 0 (its output is v_0), and each
    (batch, query head) tensor's tolerance is 2e-3 times the largest oracle
    element among its sampled rows: a lower bound of the tensor's maximum,
    so the check is at least as strict as the contract."""
    import torch
    k_ = kve()
    dev = torch.device("cuda")
    b, H, G, n, S, W, B = case
    d, kk = 128, B - S - W
    print(f"[prefill-full] {case}", flush=True)
    shape = k_.Shape(b, H, G, d, n, k_.BF16)
    c = k_.CacheTensors.empty(shape, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(n)
    c.k.copy_(torch.randn(c.k.shape, generator=g, device=dev).to(torch.bfloat16))
    c.v.copy_(torch.randn(c.v.shape, generator=g, device=dev).to(torch.bfloat16))
    c.score.copy_(torch.randn(c.score.shape, generator=g, device=dev))
    q = torch.randn((b, H * G, n, d), generator=g, device=dev).to(torch.bfloat16)
    pol = k_.Policy(B, S, W, 1)
    rank = torch.empty((b, H, n), dtype=torch.int32, device=dev)
    tau = torch.empty_like(rank)
    out = torch.empty((b, H * G, n, d), device=dev)
    lse = torch.empty((b, H * G, n), device=dev)
    k_.kve_prefill_select(shape, pol, c, n, rank, tau)
    k_.kve_prefill_attn(shape, pol, c, n, rank, tau, q, out, lse)
    torch.cuda.synchronize()
    print("[prefill-full] kernels done", flush=True)
    rng = np.random.default_rng(n)
    qs = sorted(set(rng.integers(0, n, 24).tolist()) |
                {0, S + W + kk - 1, S + W + kk, n - 1})
    for bi in range(b):
        for h in (0, H - 1):
            s = c.score[bi, h].cpu().numpy()
            r = O.prefill_ranks(s)
            assert np.array_equal(rank[bi, h].cpu().numpy(), r)
            t_gpu = tau[bi, h].cpu().numpy()
            K = c.k[bi, h].float().cpu().numpy().astype(np.float64)
            V = c.v[bi, h].float().cpu().numpy().astype(np.float64)
            rows = {}  # query head -> [(position, gpu row, oracle row)]
            for qq in qs:
                elig = r[S:max(qq - W + 1, S)]
                t_ref = n if elig.shape[0] < kk else np.partition(elig, kk - 1)[kk - 1]
                assert t_gpu[qq] == t_ref, (bi, h, qq)
                t = np.arange(qq + 1)
                keep = t[(t < S) | (qq - t < W) | ((t <= qq - W) & (r[:qq + 1] <= t_ref))]
                for gq in (0, G - 1):
                    j = h * G + gq
                    qv = q[bi, j, qq].float().cpu().numpy().astype(np.float64)
                    o_ref, l_ref = O.decode_attention(qv[None], K[keep], V[keep])
                    o = out[bi, j, qq].cpu().numpy()
                    rows.setdefault(j, []).append((qq, o, o_ref[0]))
                    assert abs(float(lse[bi, j, qq]) - float(l_ref[0])) <= LSE_TOL
            for j, rs in rows.items():
                tol = ATTN_RTOL * max(np.abs(ref).max() for _, _, ref in rs)
                for qq, o, ref in rs:
                    err = np.abs(o - ref).max()
                    assert err <= tol, (bi, j, qq, err, tol)
