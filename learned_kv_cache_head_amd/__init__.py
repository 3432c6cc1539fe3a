"""libkvevict: fixed-budget KV-cache evict-and-attend decode step on MI355X.

Thin ctypes binding of the C ABI in ``include/kvevict.h`` (same entry point
names). It only marshals arguments: torch tensors supply device memory and
the current HIP stream; every step of the path runs in the library's HIP
kernels. There is no CPU fallback: if ``_lib/libkvevict.so`` is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

__all__ = [
    "KveError", "Shape", "Policy", "CacheTensors", "Scorer", "DecodeState",
    "load_library", "library_path", "kve_version", "kve_status_str",
    "kve_workspace_bytes", "kve_append", "kve_score",
    "kve_select_evict", "kve_compact", "kve_decode_attn", "kve_step",
    "F32", "BF16", "ACT_RELU", "ACT_SILU",
    "SCORER_MLP_KV", "SCORER_GATE_HIDDEN", "SCORER_MLSTM", "SCORER_SINK_GATE",
    "kve_scorer_state_bytes", "alloc_workspace", "LayerStep",
    "kve_prefill_workspace_bytes", "kve_prefill_select", "kve_prefill_attn",
    "kve_prefill_attn_workspace_bytes",
]

F32, BF16 = 0, 1
ACT_RELU, ACT_SILU = 0, 1
SCORER_MLP_KV, SCORER_GATE_HIDDEN, SCORER_MLSTM, SCORER_SINK_GATE = 0, 1, 2, 3

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_PKG, "_lib", "libkvevict.so")


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class _Policy(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_int32), ("sinks", ctypes.c_int32),
                ("window", ctypes.c_int32), ("evict_len", ctypes.c_int32),
                ("log_gamma", ctypes.c_void_p), ("gumbel", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("score", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("scorer_state", ctypes.c_void_p)]


class _Scorer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("act", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("in_dim", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("w1", ctypes.c_void_p),
                ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("delay", ctypes.c_int32),
                ("n_sink", ctypes.c_int32)]


class _State(ctypes.Structure):
    _fields_ = [("len", ctypes.c_int32), ("scored_upto", ctypes.c_int32),
                ("next_position", ctypes.c_int32), ("evicted", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "kve_version": (_I, []),
    "kve_status_str": (ctypes.c_char_p, [_I]),
    "kve_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Shape), _I]),
    "kve_scorer_state_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Shape),
                                                 ctypes.POINTER(_Scorer)]),
    "kve_append": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Cache), _I,
                        _I, _P, _P, _P]),
    "kve_score": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Scorer),
                       ctypes.POINTER(_Cache), _I, _I, _P, _P]),
    "kve_select_evict": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Policy),
                              ctypes.POINTER(_Cache), _I, _I, _P, _P]),
    "kve_compact": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Cache), _I,
                         _P, _I, _P]),
    "kve_decode_attn": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Cache),
                             _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "kve_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Shape),
                                                      _I]),
    "kve_prefill_select": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Policy),
                                ctypes.POINTER(_Cache), _I, _P, _P, _P,
                                ctypes.c_size_t, _P]),
    "kve_prefill_attn_workspace_bytes": (ctypes.c_size_t, [
        ctypes.POINTER(_Shape), ctypes.POINTER(_Policy), _I]),
    "kve_prefill_attn": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Policy),
                              ctypes.POINTER(_Cache), _I, _P, _P, _P, _P, _P,
                              _P, ctypes.c_size_t, _P]),
    "kve_step": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Policy),
                      ctypes.POINTER(_Scorer), ctypes.POINTER(_Cache),
                      ctypes.POINTER(_State), _P, _P, _P, _P, _P, _P, _P, _P,
                      _P, ctypes.c_size_t, _P]),
    "kve_step_noalloc": (_I, [ctypes.POINTER(_Shape), ctypes.POINTER(_Policy),
                              ctypes.POINTER(_Scorer), ctypes.POINTER(_Cache),
                              ctypes.POINTER(_State), _P, _P, _P, _P, _P, _P,
                              _P, _P, _P]),
}

# Bytes of the device scratch array of kve_step_noalloc (include/kvevict.h).
NOALLOC_SCRATCH_BYTES = 2 << 20

_lib = None


_lib_path = None


def load_library(path: Optional[str] = None):
    """Load libkvevict.so (built by ``__graft_entry__.build()``), or the
    build at ``path``; every call of this module then goes to it. One process
    holds one build: two copies of the library's device code in one process
    fail to launch, so asking for a second path raises."""
    global _lib, _lib_path
    p = os.path.abspath(path or library_path())
    if _lib is not None:
        if path is None or p == _lib_path:
            return _lib
        raise RuntimeError(
            f"libkvevict is already loaded from {_lib_path}; one process "
            f"cannot also load {p}")
    if not os.path.exists(p):
        raise RuntimeError(
            f"libkvevict is not built ({p} missing); run "
            "__graft_entry__.build() first")
    # PyTorch ships its own HIP runtime (libamdhip64.so, soname
    # libamdhip64.so.7). Loaded after torch, the library links against that
    # copy; loaded before it, the library would bind the system's runtime and
    # torch would then load a second one, whose device memory and streams
    # the library's launches cannot use.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib, _lib_path = lib, p
    return lib


class KveError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kve_status_str(status)} (status {status})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KveError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _dev(t, nbytes: int, name: str, optional: bool = False) -> Optional[int]:
    """Pointer of a device tensor that must hold at least ``nbytes``
    contiguous bytes. The C ABI takes bare pointers and cannot see buffer
    sizes, so a tensor that is too small, strided or on the host is refused
    here instead of reaching a kernel."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name}: a device tensor is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, needs at least {nbytes}")
    return t.data_ptr()


def _check_cache(shape: "Shape", cache: "CacheTensors", kv: bool = True,
                 score: bool = True, pos: bool = True) -> None:
    """The cache tensors a call reads or writes (kv: K and V)."""
    rows = shape.batch * shape.n_kv_heads * shape.capacity
    eb = 4 if shape.kv_dtype == F32 else 2
    if kv:
        _dev(cache.k, rows * shape.head_dim * eb, "cache.k")
        _dev(cache.v, rows * shape.head_dim * eb, "cache.v")
    if score:
        _dev(cache.score, rows * 4, "cache.score")
    if pos:
        _dev(cache.pos, rows * 4, "cache.pos")


def _check_policy(shape: "Shape", policy: "Policy") -> None:
    _dev(policy.log_gamma, shape.n_kv_heads * 4, "policy.log_gamma", True)
    _dev(policy.gumbel, shape.batch * shape.n_kv_heads * shape.capacity * 4,
         "policy.gumbel", True)


def _eb(shape: "Shape") -> int:
    return 4 if shape.kv_dtype == F32 else 2


def _check_scorer(shape: "Shape", sc: "Scorer") -> None:
    """Weight buffers large enough for the scorer kind (layouts as in
    kvevict.h)."""
    H, G, n = shape.n_kv_heads, shape.group, sc.in_dim
    web = 4 if sc.wdtype == F32 else 2
    if sc.kind == SCORER_MLP_KV:
        _dev(sc.w1, H * sc.hidden * n * web, "scorer.w1")
        _dev(sc.b1, H * sc.hidden * 4, "scorer.b1", True)
        _dev(sc.w2, H * sc.hidden * 4, "scorer.w2")
        _dev(sc.b2, H * 4, "scorer.b2", True)
    elif sc.kind == SCORER_GATE_HIDDEN:
        _dev(sc.w1, H * n * web, "scorer.w1")
        _dev(sc.b1, H * 4, "scorer.b1", True)
    elif sc.kind == SCORER_MLSTM:
        _dev(sc.w1, H * (3 * sc.hidden + 2) * n * web, "scorer.w1")
        _dev(sc.b1, H * 2 * 4, "scorer.b1", True)
        _dev(sc.w2, H * sc.hidden * 4, "scorer.w2")
        _dev(sc.b2, H * 4, "scorer.b2", True)
    elif sc.kind == SCORER_SINK_GATE:
        _dev(sc.w1, (H * 16 + H * G * 16) * n * web, "scorer.w1")
        _dev(sc.b1, 32 * 4, "scorer.b1", True)
        _dev(sc.w2, sc.n_sink * 16 * 4, "scorer.w2", sc.n_sink == 0)
        _dev(sc.b2, H * G * 4, "scorer.b2", True)


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---------------------------------------------------------------------------
# Host-side descriptors
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    batch: int
    n_kv_heads: int
    group: int
    head_dim: int
    capacity: int
    kv_dtype: int  # F32 or BF16

    def c(self) -> _Shape:
        return _Shape(self.batch, self.n_kv_heads, self.group, self.head_dim,
                      self.capacity, self.kv_dtype)

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.kv_dtype == F32 else torch.bfloat16


@dataclass(frozen=True)
class Policy:
    """Budget B, sinks S, window W, eviction length L; optional per-KV-head
    float32 log decay factors (a device tensor [n_kv_heads]); optional
    float32 Gumbel noise per cache slot (a device tensor
    [batch][n_kv_heads][capacity]) for stochastic eviction."""
    budget: int
    sinks: int
    window: int
    evict_len: int
    log_gamma: object = None
    gumbel: object = None

    def c(self) -> _Policy:
        return _Policy(self.budget, self.sinks, self.window, self.evict_len,
                       _ptr(self.log_gamma), _ptr(self.gumbel))


class CacheTensors:
    """Device tensors of one layer's cache (layouts as in kvevict.h);
    ``scorer_state`` is the stateful scorer's recurrent state or None."""

    def __init__(self, k, v, score, pos, scorer_state=None):
        self.k, self.v, self.score, self.pos = k, v, score, pos
        self.scorer_state = scorer_state

    @classmethod
    def empty(cls, shape: Shape, device="cuda"):
        import torch
        b, H, cap, d = (shape.batch, shape.n_kv_heads, shape.capacity,
                        shape.head_dim)
        dt = shape.torch_dtype
        return cls(torch.zeros((b, H, cap, d), dtype=dt, device=device),
                   torch.zeros((b, H, cap, d), dtype=dt, device=device),
                   torch.zeros((b, H, cap), dtype=torch.float32, device=device),
                   torch.zeros((b, H, cap), dtype=torch.int32, device=device))

    def attach_scorer_state(self, shape: "Shape", scorer: "Scorer"):
        """Allocate an empty (zeroed) recurrent state for a stateful scorer;
        returns it."""
        import torch
        n = kve_scorer_state_bytes(shape, scorer)
        if n == 0:
            raise ValueError("scorer has no recurrent state for this shape")
        self.scorer_state = torch.zeros(n // 4, dtype=torch.float32,
                                        device=self.k.device)
        return self.scorer_state

    def c(self) -> _Cache:
        return _Cache(_ptr(self.k), _ptr(self.v), _ptr(self.score),
                      _ptr(self.pos), _ptr(self.scorer_state))


class Scorer:
    """Scorer weights on the device plus their descriptor."""

    def __init__(self, kind: int, w1, b1=None, w2=None, b2=None,
                 act: int = ACT_RELU, hidden: int = 0, in_dim: int = 0,
                 wdtype: Optional[int] = None, delay: int = 0,
                 n_sink: int = 0):
        import torch
        self.kind, self.act, self.delay, self.n_sink = kind, act, delay, n_sink
        self.w1, self.b1, self.w2, self.b2 = w1, b1, w2, b2
        self.hidden, self.in_dim = hidden, in_dim
        if wdtype is None:
            wdtype = F32 if w1.dtype == torch.float32 else BF16
        self.wdtype = wdtype

    @classmethod
    def mlp(cls, w1, w2, b1=None, b2=None, act: int = ACT_RELU):
        """w1 [H][hidden][2d], w2 [H][hidden], b1 [H][hidden], b2 [H]."""
        return cls(SCORER_MLP_KV, w1, b1, w2, b2, act=act,
                   hidden=w1.shape[1], in_dim=w1.shape[2])

    @classmethod
    def gate(cls, w, b=None):
        """w [H][D] bf16, b [H] float32."""
        return cls(SCORER_GATE_HIDDEN, w, b, in_dim=w.shape[1])

    @classmethod
    def mlstm(cls, w, a, gate_b=None, b=None, delay: int = 0):
        """Stateful mLSTM scorer: w [H][3P+2][2d] bf16 (rows of W_q, W_k,
        W_v, then w_i, w_f), a [H][P] float32 read-out, gate_b [H][2]
        float32 (b_i, b_f), b [H] float32; delay = the window W."""
        return cls(SCORER_MLSTM, w, gate_b, a, b, hidden=a.shape[1],
                   in_dim=w.shape[2], delay=delay)

    @classmethod
    def sink_gate(cls, w, sinks, norm=None, b=None):
        """Low-rank sink-attention gate: w [H*16 + H*G*16][D] bf16 (rows of
        W_k then W_q), sinks [S][16] float32, norm [32] float32 (k then q
        normalisation weights), b [H*G] float32."""
        return cls(SCORER_SINK_GATE, w, norm, sinks, b, hidden=16,
                   in_dim=w.shape[1], n_sink=sinks.shape[0])

    def c(self) -> _Scorer:
        return _Scorer(self.kind, self.act, self.wdtype, self.in_dim,
                       self.hidden, _ptr(self.w1), _ptr(self.b1),
                       _ptr(self.w2), _ptr(self.b2), self.delay, self.n_sink)


@dataclass
class DecodeState:
    len: int
    scored_upto: int
    next_position: int
    evicted: int = 0


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def kve_version() -> int:
    return load_library().kve_version()


def kve_status_str(status: int) -> str:
    return load_library().kve_status_str(status).decode()


def kve_workspace_bytes(shape: Shape, max_len: int) -> int:
    cs = shape.c()
    return load_library().kve_workspace_bytes(ctypes.byref(cs), max_len)


def kve_scorer_state_bytes(shape: Shape, scorer: Scorer) -> int:
    cs, csc = shape.c(), scorer.c()
    return load_library().kve_scorer_state_bytes(ctypes.byref(cs),
                                                 ctypes.byref(csc))


def alloc_workspace(shape: Shape, max_len: int, device="cuda"):
    """Allocate (torch) a workspace for caches of up to max_len entries."""
    import torch
    n = kve_workspace_bytes(shape, max_len)
    if n == 0:
        raise ValueError("invalid shape for workspace")
    return torch.empty((n + 3) // 4, dtype=torch.int32, device=device)


def kve_append(shape: Shape, cache: CacheTensors, slot: int, position: int,
               k_new, v_new, stream=None) -> None:
    _check_cache(shape, cache, score=False)
    row = shape.batch * shape.n_kv_heads * shape.head_dim * _eb(shape)
    cs, cc = shape.c(), cache.c()
    _check(load_library().kve_append(
        ctypes.byref(cs), ctypes.byref(cc), slot, position,
        _dev(k_new, row, "k_new"), _dev(v_new, row, "v_new"),
        _stream(stream)), "kve_append")


def kve_score(shape: Shape, scorer: Scorer, cache: CacheTensors,
              slot_begin: int, slot_end: int, hidden=None,
              stream=None) -> None:
    on_kv = scorer.kind in (SCORER_MLP_KV, SCORER_MLSTM)
    _check_cache(shape, cache, kv=on_kv, pos=scorer.kind == SCORER_MLSTM)
    _check_scorer(shape, scorer)
    if scorer.kind == SCORER_MLSTM:
        _dev(cache.scorer_state, kve_scorer_state_bytes(shape, scorer),
             "cache.scorer_state")
    rows = max(slot_end - slot_begin, 0)
    cs, csc, cc = shape.c(), scorer.c(), cache.c()
    _check(load_library().kve_score(
        ctypes.byref(cs), ctypes.byref(csc), ctypes.byref(cc), slot_begin,
        slot_end, _dev(hidden, shape.batch * rows * scorer.in_dim * 2,
                       "hidden", True), _stream(stream)), "kve_score")


def kve_select_evict(shape: Shape, policy: Policy, cache: CacheTensors,
                     length: int, n_keep: int, keep_slots,
                     stream=None) -> None:
    _check_cache(shape, cache, kv=False)
    _check_policy(shape, policy)
    cs, cp, cc = shape.c(), policy.c(), cache.c()
    keep = _dev(keep_slots, shape.batch * shape.n_kv_heads * max(n_keep, 0) * 4,
                "keep_slots")
    _check(load_library().kve_select_evict(
        ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(cc), length, n_keep,
        keep, _stream(stream)), "kve_select_evict")


def kve_compact(shape: Shape, cache: CacheTensors, length: int, keep_slots,
                n_keep: int, stream=None) -> None:
    _check_cache(shape, cache)
    cs, cc = shape.c(), cache.c()
    keep = _dev(keep_slots, shape.batch * shape.n_kv_heads * max(n_keep, 0) * 4,
                "keep_slots")
    _check(load_library().kve_compact(
        ctypes.byref(cs), ctypes.byref(cc), length, keep, n_keep,
        _stream(stream)), "kve_compact")


def _check_attn_io(shape: Shape, q, out, lse) -> None:
    hq = shape.batch * shape.n_kv_heads * shape.group
    _dev(q, hq * shape.head_dim * _eb(shape), "q")
    _dev(out, hq * shape.head_dim * 4, "out")
    _dev(lse, hq * 4, "lse", True)


def kve_decode_attn(shape: Shape, cache: CacheTensors, length: int, q, out,
                    lse, ws, stream=None) -> None:
    _check_cache(shape, cache, score=False, pos=False)
    _check_attn_io(shape, q, out, lse)
    cs, cc = shape.c(), cache.c()
    _check(load_library().kve_decode_attn(
        ctypes.byref(cs), ctypes.byref(cc), length, _ptr(q), _ptr(out),
        _ptr(lse), _dev(ws, 0, "ws", True),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)), "kve_decode_attn")


def _check_step_args(shape, policy, scorer, cache, k_new, v_new, q, out, lse,
                     keep_slots, ws, hidden_new, hidden_buf,
                     need_ws: bool = True) -> None:
    _check_cache(shape, cache)
    _check_policy(shape, policy)
    _check_scorer(shape, scorer)
    if scorer.kind == SCORER_MLSTM:
        _dev(cache.scorer_state, kve_scorer_state_bytes(shape, scorer),
             "cache.scorer_state")
    _check_attn_io(shape, q, out, lse)
    row = shape.batch * shape.n_kv_heads * shape.head_dim * _eb(shape)
    _dev(k_new, row, "k_new")
    _dev(v_new, row, "v_new")
    _dev(keep_slots, shape.batch * shape.n_kv_heads * policy.budget * 4,
         "keep_slots")
    if need_ws:
        _dev(ws, 0, "ws")
    _dev(hidden_new, shape.batch * scorer.in_dim * 2, "hidden_new", True)
    _dev(hidden_buf, shape.batch * policy.evict_len * scorer.in_dim * 2,
         "hidden_buf", True)


def kve_step(shape: Shape, policy: Policy, scorer: Scorer,
             cache: CacheTensors, state: DecodeState, k_new, v_new, q, out,
             lse, keep_slots, ws, hidden_new=None, hidden_buf=None,
             stream=None) -> DecodeState:
    """One decode step of one layer; updates and returns ``state``."""
    _check_step_args(shape, policy, scorer, cache, k_new, v_new, q, out, lse,
                     keep_slots, ws, hidden_new, hidden_buf)
    cs, cp, csc, cc = shape.c(), policy.c(), scorer.c(), cache.c()
    st = _State(state.len, state.scored_upto, state.next_position, 0)
    _check(load_library().kve_step(
        ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(csc),
        ctypes.byref(cc), ctypes.byref(st), _ptr(k_new), _ptr(v_new),
        _ptr(hidden_new), _ptr(hidden_buf), _ptr(q), _ptr(out), _ptr(lse),
        _ptr(keep_slots), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)), "kve_step")
    state.len, state.scored_upto = st.len, st.scored_upto
    state.next_position, state.evicted = st.next_position, st.evicted
    return state


def kve_step_noalloc(shape: Shape, policy: Policy, scorer: Scorer,
                     cache: CacheTensors, state: DecodeState, k_new, v_new, q,
                     out, lse, keep_slots, hidden_new=None, hidden_buf=None,
                     stream=None) -> DecodeState:
    """``kve_step`` without a workspace: the split-K partials live in the
    library's per-GPU scratch array, and the call allocates nothing. Calls
    that overlap on one GPU race (order them on one stream)."""
    _check_step_args(shape, policy, scorer, cache, k_new, v_new, q, out, lse,
                     keep_slots, None, hidden_new, hidden_buf,
                     need_ws=False)
    cs, cp, csc, cc = shape.c(), policy.c(), scorer.c(), cache.c()
    st = _State(state.len, state.scored_upto, state.next_position, 0)
    _check(load_library().kve_step_noalloc(
        ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(csc),
        ctypes.byref(cc), ctypes.byref(st), _ptr(k_new), _ptr(v_new),
        _ptr(hidden_new), _ptr(hidden_buf), _ptr(q), _ptr(out), _ptr(lse),
        _ptr(keep_slots), _stream(stream)), "kve_step_noalloc")
    state.len, state.scored_upto = st.len, st.scored_upto
    state.next_position, state.evicted = st.next_position, st.evicted
    return state


def kve_prefill_workspace_bytes(shape: Shape, length: int) -> int:
    cs = shape.c()
    return load_library().kve_prefill_workspace_bytes(ctypes.byref(cs), length)


def kve_prefill_select(shape: Shape, policy: Policy, cache: CacheTensors,
                       length: int, rank, tau, ws=None, stream=None) -> None:
    """Ranks and running top-k cutoffs of a prompt (slot s = position s).
    Allocates the scratch workspace with torch when none is given."""
    import torch
    if ws is None:
        n = kve_prefill_workspace_bytes(shape, length)
        if n == 0:
            raise ValueError("invalid shape or length for prefill selection")
        ws = torch.empty(n // 8, dtype=torch.int64, device=rank.device)
    _check_cache(shape, cache, kv=False, pos=False)
    _check_policy(shape, policy)
    per = shape.batch * shape.n_kv_heads * max(length, 0) * 4
    cs, cp, cc = shape.c(), policy.c(), cache.c()
    _check(load_library().kve_prefill_select(
        ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(cc), length,
        _dev(rank, per, "rank"), _dev(tau, per, "tau"), _dev(ws, 0, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "kve_prefill_select")


def kve_prefill_attn_workspace_bytes(shape: Shape, policy: Policy,
                                     length: int) -> int:
    cs, cp = shape.c(), policy.c()
    return load_library().kve_prefill_attn_workspace_bytes(
        ctypes.byref(cs), ctypes.byref(cp), length)


def kve_prefill_attn(shape: Shape, policy: Policy, cache: CacheTensors,
                     length: int, rank, tau, q, out, lse=None, ws=None,
                     stream=None) -> None:
    """Eq. 26 masked prefill attention; allocates the key-list workspace
    with torch when none is given."""
    import torch
    if ws is None:
        n = kve_prefill_attn_workspace_bytes(shape, policy, length)
        if n == 0:
            raise ValueError("invalid shape, policy or length")
        ws = torch.empty((n + 3) // 4, dtype=torch.int32, device=q.device)
    _check_cache(shape, cache, score=False, pos=False)
    _check_policy(shape, policy)
    n = max(length, 0)
    per = shape.batch * shape.n_kv_heads * n * 4
    hq = shape.batch * shape.n_kv_heads * shape.group * n
    cs, cp, cc = shape.c(), policy.c(), cache.c()
    _check(load_library().kve_prefill_attn(
        ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(cc), length,
        _dev(rank, per, "rank"), _dev(tau, per, "tau"),
        _dev(q, hq * shape.head_dim * 2, "q"),
        _dev(out, hq * shape.head_dim * 4, "out"),
        _dev(lse, hq * 4, "lse", True), _dev(ws, 0, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "kve_prefill_attn")


class LayerStep:
    """Repeated ``kve_step`` calls on one layer with the descriptors built
    once: per call only the tensor pointers of the new token and the outputs
    are marshalled, so a Python decode loop keeps the GPU queue fed.

    ``state`` (a DecodeState) is updated after every call, as by kve_step.
    """

    def __init__(self, shape: Shape, policy: Policy, scorer: Scorer,
                 cache: CacheTensors, state: DecodeState, ws, stream=None):
        self._lib = load_library()
        self._fn = self._lib.kve_step
        self._shape, self._policy = shape.c(), policy.c()
        self._scorer, self._cache = scorer.c(), cache.c()
        self._st = _State(state.len, state.scored_upto, state.next_position, 0)
        self._refs = (ctypes.byref(self._shape), ctypes.byref(self._policy),
                      ctypes.byref(self._scorer), ctypes.byref(self._cache),
                      ctypes.byref(self._st))
        self._ws_ptr = _ptr(ws)
        self._ws_bytes = ws.numel() * ws.element_size()
        self._stream = _stream(stream)
        self._keepalive = (scorer, cache, ws, policy)
        self.state = state
        self.budget, self.evict_len = policy.budget, policy.evict_len
        self._args = (shape, policy, scorer, cache, ws)
        self._checked = False

    def evicts_next(self) -> bool:
        """True if the next call reaches B + L and evicts."""
        return self._st.len + 1 >= self.budget + self.evict_len

    def __call__(self, k_new, v_new, q, out, lse, keep_slots,
                 hidden_new=None, hidden_buf=None) -> int:
        """One decode step; returns 1 if it evicted, else 0. The tensors of
        the first call are checked as by ``kve_step``; later calls are
        trusted to pass tensors of the same shapes."""
        if not self._checked:
            shape, policy, scorer, cache, ws = self._args
            _check_step_args(shape, policy, scorer, cache, k_new, v_new, q,
                             out, lse, keep_slots, ws, hidden_new, hidden_buf)
            self._checked = True
        r = self._refs
        status = self._fn(r[0], r[1], r[2], r[3], r[4], k_new.data_ptr(),
                          v_new.data_ptr(), _ptr(hidden_new), _ptr(hidden_buf),
                          q.data_ptr(), out.data_ptr(), _ptr(lse),
                          keep_slots.data_ptr(), self._ws_ptr, self._ws_bytes,
                          self._stream)
        if status != 0:
            raise KveError(status, "kve_step")
        st, s = self._st, self.state
        s.len, s.scored_upto = st.len, st.scored_upto
        s.next_position, s.evicted = st.next_position, st.evicted
        return st.evicted
