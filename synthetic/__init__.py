"""Seeded synthetic inputs for the fixed-budget evict-and-attend decode step.

This module is shared by the float64 oracle (``oracle/``) and the HIP library
tests and benchmark. It holds no arithmetic of the method itself: only the
workload shapes, seeded random draws, and the one-time rounding of drawn
values to the storage dtype (bf16, round-to-nearest-even). Every consumer gets
bit-identical inputs from the same (seed, workload, layer, step, tensor) key.

Workload shapes follow the model shapes the pages name: Qwen3-4B (36 layers,
8 KV heads, 32 query heads, head_dim 128; ForesightKV summary page, "Main
findings", 4.5 GB bf16 cache at 32K) and Qwen2.5-14B (48 layers, 8 KV heads,
head_dim 128, 192 KiB per token; KV-Kaizen, section 1 and section 2.1). The
policy knobs (sinks S, window W, budget B, eviction length L) follow KVpop
section 3 Eq. (1) and Table 3, Fast KVzip Appendix A.5 and the ForesightKV
summary ("Methodology in plain English").
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "rng_for", "round_to_bf16_bits",
    "bf16_bits_to_f32", "draw_rows", "draw_mlp_weights", "draw_gate_weights",
    "draw_mlstm_weights", "draw_sink_gate_weights",
    "initial_context", "step_inputs", "TENSOR_IDS", "gumbel_noise",
]


@dataclass(frozen=True)
class Workload:
    """Shape and policy of one synthetic decode workload."""

    cfg_id: int
    name: str
    batch: int
    n_kv: int          # KV heads H
    group: int         # query heads per KV head G
    head_dim: int      # d
    kv_dtype: str      # "f32" or "bf16" (K, V, Q and new rows)
    n0: int            # initial context length (prefill)
    sinks: int         # S
    window: int        # W
    budget: int        # B
    evict_len: int     # L
    steps: int         # decode steps
    layers: int
    scorer: str        # "mlp" ([k;v] MLP), "gate" (hidden-state gate),
                       # "sink_gate" (low-rank sink-attention gate on hidden
                       # states) or "mlstm" (stateful scorer over [k;v])
    hidden: int        # MLP hidden width, gate input dim D, or the mLSTM
                       # projection width P = d / 2
    act: str           # "relu" or "silu" (MLP only)
    structured: bool   # low-rank shared direction + heavy-hitter tokens
    heavy_frac: float = 0.01
    heavy_scale: float = 4.0

    @property
    def n_q(self) -> int:
        return self.n_kv * self.group

    @property
    def in_dim(self) -> int:
        return (self.hidden if self.scorer in ("gate", "sink_gate")
                else 2 * self.head_dim)

    @property
    def capacity(self) -> int:
        return max(self.n0, self.budget + self.evict_len)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    @property
    def wdtype(self) -> str:
        return self.kv_dtype


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-1layer-fp32", batch=1, n_kv=2, group=2, head_dim=64,
                kv_dtype="f32", n0=512, sinks=4, window=64, budget=192,
                evict_len=1, steps=64, layers=1, scorer="mlp", hidden=32,
                act="relu", structured=False),
    2: Workload(2, "qwen3-4b-1layer-b16", batch=16, n_kv=8, group=4,
                head_dim=128, kv_dtype="bf16", n0=8192, sinks=4, window=128,
                budget=1024, evict_len=128, steps=256, layers=1, scorer="mlp",
                hidden=64, act="relu", structured=True),
    3: Workload(3, "qwen3-4b-36layer-b8-B2048", batch=8, n_kv=8, group=4,
                head_dim=128, kv_dtype="bf16", n0=8192, sinks=4, window=256,
                budget=2048, evict_len=256, steps=24576, layers=36,
                scorer="mlp", hidden=64, act="relu", structured=False),
    4: Workload(4, "qwen3-4b-36layer-b96-B1024", batch=96, n_kv=8, group=4,
                head_dim=128, kv_dtype="bf16", n0=8192, sinks=4, window=128,
                budget=1024, evict_len=128, steps=512, layers=36,
                scorer="mlp", hidden=64, act="relu", structured=False),
    5: Workload(5, "qwen2.5-14b-48layer-131k-gate", batch=1, n_kv=8, group=5,
                head_dim=128, kv_dtype="bf16", n0=131072, sinks=4, window=512,
                budget=39321, evict_len=64, steps=512, layers=48,
                scorer="gate", hidden=5120, act="relu", structured=False),
}


def workload(cfg_id: int, **overrides) -> Workload:
    """Return workload ``cfg_id``, optionally with fields replaced (smaller
    test sizes keep the same structure)."""
    w = WORKLOADS[cfg_id]
    return replace(w, **overrides) if overrides else w


# Tensor ids used in the seed key; fixed so that streams never collide.
TENSOR_IDS = {
    "k0": 1, "v0": 2, "k_new": 3, "v_new": 4, "q": 5, "heavy": 6,
    "dir_k": 7, "dir_v": 8, "w1": 9, "w2": 10, "b1": 11, "b2": 12,
    "gate_w": 13, "hidden0": 14, "hidden_new": 15, "misc": 16,
    "mlstm_w": 17, "mlstm_gb": 18, "mlstm_a": 19,
    "sg_w": 20, "sg_norm": 21, "sg_sinks": 22, "sg_b": 23,
}


def rng_for(seed: int, cfg_id: int, layer: int, step: int,
            tensor: str) -> np.random.Generator:
    """PCG64 stream keyed by (seed, workload, layer, step, tensor).

    ``step`` is -1 for the initial context and layer-constant tensors.
    """
    key = [int(seed), int(cfg_id), int(layer), int(step) + 1,
           TENSOR_IDS[tensor]]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def round_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. Inputs must be finite.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


class Stored:
    """A drawn tensor in its storage dtype.

    ``bits`` holds the raw storage (uint16 bf16 patterns or float32 values)
    and ``f64`` the exact float64 value of every stored element.
    """

    def __init__(self, values_f32: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = round_to_bf16_bits(values_f32)
            self.f64 = bf16_bits_to_f32(self.bits).astype(np.float64)
        elif dtype == "f32":
            self.bits = np.ascontiguousarray(values_f32, dtype=np.float32)
            self.f64 = self.bits.astype(np.float64)
        else:
            raise ValueError(dtype)

    @property
    def shape(self):
        return self.bits.shape

    def torch(self, device=None):
        """A torch tensor holding exactly the stored values."""
        import torch
        if self.dtype == "bf16":
            t = torch.from_numpy(self.bits.view(np.int16).copy()).view(
                torch.bfloat16)
        else:
            t = torch.from_numpy(self.bits.copy())
        return t.to(device) if device is not None else t


def _directions(w: Workload, seed: int, layer: int, which: str) -> np.ndarray:
    """One unit vector per KV head (the shared low-rank direction)."""
    g = rng_for(seed, w.cfg_id, layer, -1, which)
    u = g.standard_normal((w.n_kv, w.head_dim))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def draw_rows(w: Workload, seed: int, layer: int, step: int, tensor: str,
              n_tokens: int, heavy: Optional[np.ndarray]) -> np.ndarray:
    """K or V rows [batch][n_kv][n_tokens][d] as float32 (before rounding).

    Unstructured workloads draw i.i.d. N(0, 1). Structured workloads add
    sqrt(d) times a per-head unit direction to every row, and multiply the
    rows of heavy-hitter tokens (``heavy`` mask [batch][n_tokens]) by
    ``heavy_scale`` in every head.
    """
    g = rng_for(seed, w.cfg_id, layer, step, tensor)
    z = g.standard_normal((w.batch, w.n_kv, n_tokens, w.head_dim))
    if w.structured:
        u = _directions(w, seed, layer, "dir_k" if tensor.startswith("k")
                        else "dir_v")
        z = z + np.sqrt(w.head_dim) * u[None, :, None, :]
        if heavy is not None:
            z = np.where(heavy[:, None, :, None], z * w.heavy_scale, z)
    return z.astype(np.float32)


def _heavy(w: Workload, seed: int, layer: int, step: int,
           n_tokens: int) -> Optional[np.ndarray]:
    if not w.structured:
        return None
    g = rng_for(seed, w.cfg_id, layer, step, "heavy")
    return g.random((w.batch, n_tokens)) < w.heavy_frac


def draw_mlp_weights(w: Workload, seed: int, layer: int,
                     biases: bool = False) -> dict:
    """Per-KV-head MLP scorer weights.

    w1 [H][hidden][2d] in the workload's weight dtype, N(0, 1/(2d));
    w2 [H][hidden] float32, N(0, 1/hidden); b1 [H][hidden] and b2 [H] float32
    (zero unless ``biases``, then N(0, 0.1^2)).
    """
    in_dim = 2 * w.head_dim
    g1 = rng_for(seed, w.cfg_id, layer, -1, "w1")
    w1 = g1.standard_normal((w.n_kv, w.hidden, in_dim)) / np.sqrt(in_dim)
    g2 = rng_for(seed, w.cfg_id, layer, -1, "w2")
    w2 = g2.standard_normal((w.n_kv, w.hidden)) / np.sqrt(w.hidden)
    if biases:
        b1 = 0.1 * rng_for(seed, w.cfg_id, layer, -1, "b1").standard_normal(
            (w.n_kv, w.hidden))
        b2 = 0.1 * rng_for(seed, w.cfg_id, layer, -1, "b2").standard_normal(
            (w.n_kv,))
    else:
        b1 = np.zeros((w.n_kv, w.hidden))
        b2 = np.zeros((w.n_kv,))
    return {
        "w1": Stored(w1.astype(np.float32), w.wdtype),
        "w2": Stored(w2.astype(np.float32), "f32"),
        "b1": Stored(b1.astype(np.float32), "f32"),
        "b2": Stored(b2.astype(np.float32), "f32"),
    }


def draw_gate_weights(w: Workload, seed: int, layer: int,
                      bias: bool = False) -> dict:
    """Per-KV-head gate weights w [H][D] (bf16, N(0, 1/D)) and bias [H]."""
    g = rng_for(seed, w.cfg_id, layer, -1, "gate_w")
    gw = g.standard_normal((w.n_kv, w.hidden)) / np.sqrt(w.hidden)
    if bias:
        b = 0.1 * rng_for(seed, w.cfg_id, layer, -1, "b1").standard_normal(
            (w.n_kv,))
    else:
        b = np.zeros((w.n_kv,))
    return {"w": Stored(gw.astype(np.float32), "bf16"),
            "b": Stored(b.astype(np.float32), "f32")}


def draw_mlstm_weights(w: Workload, seed: int, layer: int) -> dict:
    """Per-KV-head stateful-scorer weights, P = d / 2:
    w [H][3P+2][2d] bf16 (rows W_q, W_k, W_v, then w_i, w_f), N(0, 1/(2d)),
    with the W_q and W_k rows scaled by 2 so that the Hedgehog features are
    not flat; gate_b [H][2] float32: input bias N(0, 0.5^2), forget bias
    3 + N(0, 1) (a forget gate near 0.95, long memory); a [H][P] float32,
    N(0, 1/P); b [H] float32, N(0, 0.1^2)."""
    P = w.head_dim // 2
    in_dim = 2 * w.head_dim
    g = rng_for(seed, w.cfg_id, layer, -1, "mlstm_w")
    wt = g.standard_normal((w.n_kv, 3 * P + 2, in_dim)) / np.sqrt(in_dim)
    wt[:, :2 * P] *= 2.0
    gg = rng_for(seed, w.cfg_id, layer, -1, "mlstm_gb")
    gb = np.stack([0.5 * gg.standard_normal(w.n_kv),
                   3.0 + gg.standard_normal(w.n_kv)], axis=1)
    ga = rng_for(seed, w.cfg_id, layer, -1, "mlstm_a")
    a = ga.standard_normal((w.n_kv, P)) / np.sqrt(P)
    b = 0.1 * ga.standard_normal(w.n_kv)
    return {"w": Stored(wt.astype(np.float32), "bf16"),
            "gate_b": Stored(gb.astype(np.float32), "f32"),
            "a": Stored(a.astype(np.float32), "f32"),
            "b": Stored(b.astype(np.float32), "f32")}


def draw_sink_gate_weights(w: Workload, seed: int, layer: int,
                           n_sink: int = 16) -> dict:
    """Low-rank sink-attention gate of one layer, D' = 16 (Fast KVzip
    section 3.4, S = D' = 16): w [H*16 + H*G*16][D] bf16, N(0, 1/D) (rows of
    W_k, then W_q); norm [32] float32, 0.5 + U(0, 1) (k then q weights);
    sinks [S][16] float32, N(0, 1); b [H*G] float32, U(0, 1)."""
    D, H, G = w.hidden, w.n_kv, w.group
    g = rng_for(seed, w.cfg_id, layer, -1, "sg_w")
    wt = g.standard_normal((H * 16 + H * G * 16, D)) / np.sqrt(D)
    norm = 0.5 + rng_for(seed, w.cfg_id, layer, -1, "sg_norm").random(32)
    sinks = rng_for(seed, w.cfg_id, layer, -1, "sg_sinks").standard_normal(
        (n_sink, 16))
    b = rng_for(seed, w.cfg_id, layer, -1, "sg_b").random(H * G)
    return {"w": Stored(wt.astype(np.float32), "bf16"),
            "norm": Stored(norm.astype(np.float32), "f32"),
            "sinks": Stored(sinks.astype(np.float32), "f32"),
            "b": Stored(b.astype(np.float32), "f32")}


def gumbel_noise(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard Gumbel noise (numpy's generator), rounded once to float32:
    the random input of stochastic eviction."""
    return rng.gumbel(size=shape).astype(np.float32)


def initial_context(w: Workload, seed: int, layer: int) -> dict:
    """The prefill cache of one layer: positions 0..n0-1 in every head.

    Returns k0, v0 ([batch][H][n0][d], Stored) and, for the gate scorer,
    hidden0 ([batch][n0][D], bf16 Stored).
    """
    heavy = _heavy(w, seed, layer, -1, w.n0)
    out = {
        "k0": Stored(draw_rows(w, seed, layer, -1, "k0", w.n0, heavy),
                     w.kv_dtype),
        "v0": Stored(draw_rows(w, seed, layer, -1, "v0", w.n0, heavy),
                     w.kv_dtype),
    }
    if w.scorer in ("gate", "sink_gate"):
        g = rng_for(seed, w.cfg_id, layer, -1, "hidden0")
        out["hidden0"] = Stored(
            g.standard_normal((w.batch, w.n0, w.hidden)).astype(np.float32),
            "bf16")
    return out


def step_inputs(w: Workload, seed: int, layer: int, step: int) -> dict:
    """Inputs of decode step ``step`` (0-based) of one layer.

    k_new, v_new [batch][H][d]; q [batch][H*G][d] (N(0,1)); for the gate
    scorer also hidden_new [batch][D].
    """
    heavy = _heavy(w, seed, layer, step, 1)
    k = draw_rows(w, seed, layer, step, "k_new", 1, heavy)[:, :, 0, :]
    v = draw_rows(w, seed, layer, step, "v_new", 1, heavy)[:, :, 0, :]
    gq = rng_for(seed, w.cfg_id, layer, step, "q")
    q = gq.standard_normal((w.batch, w.n_q, w.head_dim)).astype(np.float32)
    out = {"k_new": Stored(k, w.kv_dtype), "v_new": Stored(v, w.kv_dtype),
           "q": Stored(q, w.kv_dtype)}
    if w.scorer in ("gate", "sink_gate"):
        g = rng_for(seed, w.cfg_id, layer, step, "hidden_new")
        out["hidden_new"] = Stored(
            g.standard_normal((w.batch, w.hidden)).astype(np.float32), "bf16")
    return out


def device_normal(shape, seed: int, key: tuple, dtype=None, device="cuda",
                  scale: float = 1.0):
    """N(0, scale^2) draws generated on the device by torch's Philox
    generator, keyed by (seed, *key); rounded once to ``dtype`` (default
    bf16). Used for the large workloads whose inputs are too big to draw on
    the host."""
    import torch
    dtype = dtype or torch.bfloat16
    ss = np.random.SeedSequence([int(seed), *[int(x) for x in key]])
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1)))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)
