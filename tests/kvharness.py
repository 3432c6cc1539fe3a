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
