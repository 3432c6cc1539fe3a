"""Shared helpers of the parity tests: move synthetic inputs to the device,
run the HIP path through the C ABI, and run the float64 oracle on the same
inputs. Used by tests and by the package smoke check only."""
from __future__ import annotations

import numpy as np

import oracle as O
import synthetic as syn

ATTN_RTOL = 2e-3      # attention: |gpu - oracle| <= 2e-3 * max|oracle out|
SCORE_ATOL = 1e-3     # scores: |gpu - oracle| <= 1e-3
LSE_ATOL = 1e-4       # lse: float32 rounding of values of magnitude <~ 30


def kve():
    import learned_kv_cache_head_amd as k
    k.load_library()
    return k


def dtype_code(w: syn.Workload) -> int:
    import learned_kv_cache_head_amd as k
    return k.F32 if w.kv_dtype == "f32" else k.BF16


def shape_of(w: syn.Workload, capacity=None):
    k = kve()
    return k.Shape(w.batch, w.n_kv, w.group, w.head_dim,
                   capacity or w.capacity, dtype_code(w))


def to_f64(t) -> np.ndarray:
    """Exact float64 values of a device tensor."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_mlp_scores(k64, v64, wts, act) -> np.ndarray:
    """Oracle float32 scores of rows k64/v64 [b][H][n][d] with per-head
    weights from synthetic.draw_mlp_weights."""
    b, H = k64.shape[:2]
    out = np.empty(k64.shape[:3], dtype=np.float32)
    for bi in range(b):
        for h in range(H):
            out[bi, h] = O.score_to_f32(O.mlp_score(
                k64[bi, h], v64[bi, h], wts["w1"].f64[h], wts["b1"].f64[h],
                wts["w2"].f64[h], wts["b2"].f64[h], act))
    return out


def oracle_gate_scores(hidden64, gw) -> np.ndarray:
    """hidden64 [b][n][D] -> float32 scores [b][H][n]."""
    b = hidden64.shape[0]
    H = gw["w"].f64.shape[0]
    out = np.empty((b, H, hidden64.shape[1]), dtype=np.float32)
    for bi in range(b):
        for h in range(H):
            out[bi, h] = O.score_to_f32(O.gate_score(
                hidden64[bi], gw["w"].f64[h], gw["b"].f64[h]))
    return out


def attn_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Assert the attention tolerance; return the relative error."""
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    rel = err / scale if scale > 0 else err
    assert rel <= ATTN_RTOL, f"{what}: attention error {rel:.3e} > {ATTN_RTOL}"
    return rel


def retained_sets_agree(gpu_pos: np.ndarray, ora_pos: np.ndarray,
                        ora_score_by_pos: dict, cut: float) -> bool:
    """End-to-end retained sets must be equal except for tokens whose oracle
    score lies within SCORE_ATOL of the cut score."""
    a, b = set(gpu_pos.tolist()), set(ora_pos.tolist())
    for t in a ^ b:
        if abs(float(ora_score_by_pos[t]) - cut) > SCORE_ATOL:
            return False
    return True


def oracle_mlstm_weights(wts: dict, h: int) -> O.MlstmWeights:
    """Head h's stateful-scorer weights (synthetic.draw_mlstm_weights) in
    the oracle's form: rows W_q, W_k, W_v, w_i, w_f of w [H][3P+2][2d]."""
    w = wts["w"].f64[h]
    P = wts["a"].f64.shape[1]
    gb = wts["gate_b"].f64[h]
    return O.MlstmWeights(w[:P], w[P:2 * P], w[2 * P:3 * P], w[3 * P],
                          w[3 * P + 1], float(gb[0]), float(gb[1]),
                          wts["a"].f64[h], float(wts["b"].f64[h]))


def mlstm_device_scorer(wts: dict, delay: int, device):
    """The library's Scorer for synthetic.draw_mlstm_weights output."""
    k = kve()
    return k.Scorer.mlstm(wts["w"].torch(device), wts["a"].torch(device),
                          gate_b=wts["gate_b"].torch(device),
                          b=wts["b"].torch(device), delay=delay)


class Tracker:
    """All tokens' K/V/score by position for every slice, plus the oracle
    layer; used to compare retained sets and recompute attention."""

    def __init__(self, w, k0, v0, s0, policy):
        self.w = w
        self.policy = policy
        self.lg = policy.log_gamma
        npos = w.n0 + w.steps
        b, H, d = w.batch, w.n_kv, w.head_dim
        self.K = np.zeros((b, H, npos, d))
        self.V = np.zeros((b, H, npos, d))
        self.S = np.zeros((b, H, npos), np.float32)
        self.K[:, :, :w.n0], self.V[:, :, :w.n0] = k0, v0
        self.S[:, :, :w.n0] = s0
        self.lay = O.OracleLayer(k0, v0, s0, policy, w.group)
        self.cut = np.full((b, H), np.nan)

    def _record_cut(self):
        """Lowest kept score among the eligible entries right after an
        eviction (positions S..P-W): the cut of the next comparison."""
        p = self.policy
        b, H = self.lay.pos.shape[:2]
        for bi in range(b):
            for h in range(H):
                m = O.eligible_mask(self.lay.pos[bi, h], p.sinks, p.window)
                if m.any():
                    key = self._key(self.lay.score[bi, h], self.lay.pos[bi, h], h)
                    self.cut[bi, h] = float(key[m].min())

    def _key(self, score32, pos, h):
        """The ranking key: score, or static priority under decay."""
        return O.static_priority(score32, pos,
                                 None if self.lg is None else self.lg[h])

    def prefill(self):
        if self.lay.prefill_compress() is not None:
            self._record_cut()

    def step(self, pos, k, v, s, delayed=None, gumbel=None):
        """Append the token at ``pos``; ``delayed`` = (u, scores [b][H])
        gives an earlier token its score (stateful scorers) before the
        eviction check; ``gumbel`` (noise by slot) makes it stochastic."""
        self.K[:, :, pos], self.V[:, :, pos], self.S[:, :, pos] = k, v, s
        self.lay.append(k, v, s)
        if delayed is not None:
            u, su = delayed
            self.S[:, :, u] = su
            self.lay.set_scores(u, su)
        if self.lay.maybe_evict(gumbel) is not None:
            self._record_cut()

    def check_and_sync(self, gpu_pos):
        """Compare the GPU's retained positions [b][H][n] with the oracle's;
        resynchronise the oracle to the GPU set on tolerated tie flips."""
        b, H, n = gpu_pos.shape
        assert n == self.lay.n, f"cache count {n} != oracle {self.lay.n}"
        for bi in range(b):
            for h in range(H):
                g = gpu_pos[bi, h]
                o = self.lay.pos[bi, h]
                if np.array_equal(g, o):
                    continue
                diff = set(g.tolist()) ^ set(o.tolist())
                for t in diff:
                    key = float(self._key(self.S[bi, h, t:t + 1],
                                          np.array([t]), h)[0])
                    assert abs(key - self.cut[bi, h]) <= SCORE_ATOL, \
                        f"slice {bi},{h}: token {t} differs"
                self.lay.K[bi, h] = self.K[bi, h, g]
                self.lay.V[bi, h] = self.V[bi, h, g]
                self.lay.score[bi, h] = self.S[bi, h, g]
                self.lay.pos[bi, h] = g


def oracle_sink_gate_weights(wts: dict, H: int, G: int) -> O.SinkGateWeights:
    """synthetic.draw_sink_gate_weights output in the oracle's form."""
    w = wts["w"].f64
    D = w.shape[1]
    return O.SinkGateWeights(w[:H * 16].reshape(H, 16, D),
                             w[H * 16:].reshape(H, G, 16, D),
                             wts["norm"].f64[:16], wts["norm"].f64[16:],
                             wts["sinks"].f64, wts["b"].f64.reshape(H, G))


def oracle_sink_gate_scores(hidden64, wts, H, G) -> np.ndarray:
    """hidden [b][n][D] -> float32 scores [b][H][n]."""
    w = oracle_sink_gate_weights(wts, H, G)
    out = np.stack([O.sink_gate_score(hidden64[bi], w).T
                    for bi in range(hidden64.shape[0])])
    return O.score_to_f32(out)
