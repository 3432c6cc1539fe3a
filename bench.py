"""Decode-step benchmark of libkvevict on one MI355X.

One step = one decode token through every attention layer of the stack for
the whole batch: per layer, ``kve_step`` appends the new K/V row, and on
every L-th step scores the pending rows (MLP over [k; v]), selects the
evicted rows and compacts the cache back to the budget B; then it runs GQA
decode attention over the retained rows. Inputs are synthetic and already
resident in HBM when the timed region starts.

Default workload: Qwen3-4B-shaped attention stack (36 layers, 8 KV heads, 32
query heads, head_dim 128, bf16 K/V/Q, float32 accumulation), batch 96,
every sequence holding a compressed cache of B = 1024 entries (S = 4 sinks,
W = 128 window, eviction length L = 128) after an 8192-token prompt that the
library itself scores, selects and compacts during set-up.

Prints one JSON line with tokens/s, the achieved bandwidth of the dominant
kernel (decode attention) against the HBM roofline, and the float64 CPU
oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, GB/s
WORKLOAD_BY_NAME = {
    "qwen3-4b-36layer-b96-B1024": 4,
    "qwen3-4b-36layer-b8-B2048": 3,
    "qwen3-4b-1layer-b16": 2,
    "qwen2.5-14b-48layer-131k-gate": 5,
    "tiny-1layer-fp32": 1,
    # the batch-96 stack at the 2K budget of the batch-8 workload (S 4,
    # W 256, L 256): the upper end of B = 1024-2048 with the chip filled
    "qwen3-4b-36layer-b96-B2048": (4, dict(
        name="qwen3-4b-36layer-b96-B2048", budget=2048, window=256,
        evict_len=256)),
}


def workload_for(name: str):
    """The synthetic workload a bench workload name stands for."""
    import synthetic as syn
    spec = WORKLOAD_BY_NAME[name]
    if isinstance(spec, tuple):
        return syn.workload(spec[0], **spec[1])
    return syn.workload(spec)
DEFAULT_WORKLOAD = "qwen3-4b-36layer-b96-B1024"
ATTN_SOURCE = os.path.join(ROOT, "learned_kv_cache_head_amd", "csrc",
                           "attention.hip")
SCORE_SOURCE = os.path.join(ROOT, "learned_kv_cache_head_amd", "csrc",
                            "score.hip")
METRIC = ("evict+decode tokens/s at budget B and achieved HBM GB/s vs "
          "MI355X peak")


def achievable_copy_gbps(dev) -> float:
    """Best of three timed 1 GiB device-to-device copies (1 GiB read + 1 GiB
    written), in GB/s: the achievable-bandwidth reference."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


def achievable_read_gbps(dev, gib: int = 4) -> float:
    """Best of three timed reads of a `gib` GiB device buffer by the
    read-only reference kernel (libkvebench.so: 16-byte non-temporal loads,
    the load form of the attention's K/V stream, nothing written but one
    word per workgroup), in GB/s: the read ceiling a streaming kernel can be
    held against."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "learned_kv_cache_head_amd", "_lib",
                                   "libkvebench.so"))
    lib.kvebench_read.restype = ctypes.c_int
    lib.kvebench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.kvebench_read_blocks.restype = ctypes.c_size_t
    lib.kvebench_read_blocks.argtypes = [ctypes.c_size_t]
    nbytes = gib << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    sink = torch.empty(int(lib.kvebench_read_blocks(nbytes)),
                       dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def read():
        rc = lib.kvebench_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"kvebench_read failed ({rc})")

    read()
    best = 0.0
    for _ in range(3):
        e0, e1 = (torch.cuda.Event(enable_timing=True),
                  torch.cuda.Event(enable_timing=True))
        e0.record()
        read()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    torch.cuda.empty_cache()
    return best


def issue_probe(dev) -> dict:
    """How far MFMAs and vector ALU work overlap on one SIMD (libkvebench.so,
    issue_kernel): workgroups of 8 waves, waves w and w + 4 on one SIMD.
    Per SIMD-iteration a wave running MFMAs issues 8 independent
    v_mfma_f32_16x16x32_bf16; a vector wave 32 float32 FMAs (or 32 v_exp_f32)
    over 8 chains. Reports ns per SIMD-iteration; when the two overlap, the
    combined modes take the longer of the two parts, when they serialise,
    their sum."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "learned_kv_cache_head_amd", "_lib",
                                   "libkvebench.so"))
    lib.kvebench_issue.restype = ctypes.c_int
    lib.kvebench_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = 4 * cus, 4000
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    simd_iters = blocks * 4 * iters / (cus * 4)
    modes = [("mfma", 1), ("fma", 2), ("mfma_and_fma_two_waves", 3),
             ("mfma_and_fma_one_wave", 5), ("exp", 10),
             ("mfma_and_exp_two_waves", 11), ("mfma_and_exp_one_wave", 13)]
    res = {}
    for name, mode in modes:
        best = None
        for _ in range(3):
            e0, e1 = (torch.cuda.Event(enable_timing=True),
                      torch.cuda.Event(enable_timing=True))
            e0.record()
            rc = lib.kvebench_issue(mode, blocks, iters, out.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"kvebench_issue failed ({rc})")
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        res[name] = round(best * 1e6 / simd_iters, 1)
    return {"ns_per_simd_iteration": res,
            "per_iteration": {"mfma": "8 x v_mfma_f32_16x16x32_bf16",
                              "fma": "32 x v_fma_f32", "exp": "32 x v_exp_f32"},
            "workgroups": blocks, "iterations": iters}


def library_reference(dev) -> dict:
    """The vendor libraries behind torch at the shapes of two kernels here,
    as context for their MFMA fractions: the bf16 GEMM of the sink gate's
    projections (131072 x 5120 hidden states by 768 weight rows) and torch's
    fused attention (scaled_dot_product_attention) over batch 8, 32 heads,
    8192 positions, d 128, dense causal and dense non-causal, in TFLOP/s
    (best of three)."""
    import torch
    import torch.nn.functional as F
    peak = MFMA_BF16_PEAK_TFLOPS

    def best_ms(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = (torch.cuda.Event(enable_timing=True),
                      torch.cuda.Event(enable_timing=True))
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    g = torch.Generator(device=dev).manual_seed(5)
    x = torch.randn((131072, 5120), generator=g, device=dev).to(torch.bfloat16)
    w = torch.randn((768, 5120), generator=g, device=dev).to(torch.bfloat16)
    ms = best_ms(lambda: x @ w.t())
    fl = 2 * 131072 * 768 * 5120
    out = {"gemm_131072x768x5120_bf16": {"ms": round(ms, 3),
                                          "tflops": round(fl / ms / 1e9, 1),
                                          "frac": round(fl / ms / 1e9 / peak, 3)}}
    del x, w
    b, h, n, d = 8, 32, 8192, 128
    q, k, v = (torch.randn((b, h, n, d), generator=g, device=dev)
               .to(torch.bfloat16) for _ in range(3))
    for causal in (True, False):
        ms = best_ms(lambda: F.scaled_dot_product_attention(q, k, v,
                                                            is_causal=causal))
        pairs = n * (n + 1) // 2 if causal else n * n
        fl = 4 * d * pairs * b * h
        out[f"sdpa_b8_h32_n8192_d128_{'causal' if causal else 'dense'}"] = {
            "ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
            "frac": round(fl / ms / 1e9 / peak, 3)}
    del q, k, v
    torch.cuda.empty_cache()
    return out


def calib_copy(dev) -> None:
    """A plain elementwise copy of known size (1 GiB read, 1 GiB written),
    the reference that scales the HBM byte counters."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes (what the method has to move; no dense-cache bytes)
# ---------------------------------------------------------------------------

def attn_launch_bytes(w, n: int, fused_append: bool) -> int:
    """Bytes one decode-attention launch must move over all (batch, KV head)
    slices at n retained rows (n counts the new row when the append is
    fused): the n K and V rows, the q rows of the group, the float32 output
    rows; with the fused append also the new row's store and position."""
    d, e, G = w.head_dim, w.elem_bytes, w.group
    per = n * 2 * d * e + G * d * e + G * d * 4
    if fused_append:
        per += 2 * d * e + 4  # new K/V row written into the cache + position
    return w.batch * w.n_kv * per


def mlstm_state_bytes(w) -> int:
    """Recurrent state of one slice: C [d][d/2] and z [d] float32 plus one
    64-float block (log scale, token count)."""
    d = w.head_dim
    return (d * (d // 2) + d + 64) * 4


def score_bytes(w, scorer: str) -> int:
    """Bytes of one layer's buffered scoring of L pending rows.
    MLP: the L rows read, L scores written, per-head weights once.
    mLSTM: the L absorbed rows and the L read-out rows read, L scores
    written, the state read and written once, the slot lookup of the first
    W read-outs (ceil(W/32) scans of the B older positions), per-head
    weights once."""
    d, e, L, hid = w.head_dim, w.elem_bytes, w.evict_len, w.hidden
    slices = w.batch * w.n_kv
    if scorer == "gate":
        # the L buffered hidden states read, L scores written, weights once
        return w.batch * L * (w.hidden * 2) + slices * L * 4 + w.n_kv * w.hidden * 2
    if scorer == "mlstm":
        P = d // 2
        scans = -(-min(w.window, L) // 32) if w.window else 0
        per = (2 * L * 2 * d * e + L * 4 + 2 * mlstm_state_bytes(w)
               + scans * w.budget * 4)
        return slices * per + w.n_kv * ((3 * P + 2) * 2 * d * e + 4 * P + 12)
    return slices * (L * 2 * d * e + L * 4) + w.n_kv * (hid * 2 * d * e + hid * 4)


def evict_extra_bytes(w, n_before: int, moved: int, scorer: str = "mlp") -> int:
    """Bytes of an evicting step besides its attention launch, one layer:
    append (new row read + stored + position), scorer (``score_bytes``),
    select (candidate scores read, kept slots written), compaction (each
    moved row's K, V, score, position read and written). ``moved`` counts
    moved rows over all slices."""
    d, e = w.head_dim, w.elem_bytes
    slices = w.batch * w.n_kv
    append = slices * (2 * d * e * 2 + 4)
    score = score_bytes(w, scorer)
    cand = n_before - w.sinks - w.window
    select = slices * (cand * 8 + w.budget * 4)
    compact = moved * 2 * (2 * d * e + 8)
    return append + score + select + compact


def compress_summary(w, stack, scorer: str) -> dict:
    """Per-layer time and bytes of the one-shot prompt compression that
    set-up runs in every layer (score all n0 prompt tokens, select B, compact
    in place): median over the layers after the first, from HIP events on
    the launch stream. Bytes: scoring reads every prompt row (the K and V
    rows for the MLP scorer, the hidden states for the gate) and writes a
    score per row and KV head; select reads each entry's score and position
    and writes B kept slots; compaction reads and writes each moved row."""
    import statistics
    d, e = w.head_dim, w.elem_bytes
    slices = w.batch * w.n_kv
    if scorer == "gate":
        score_b = w.batch * w.n0 * w.hidden * 2 + slices * w.n0 * 4 + \
            w.n_kv * w.hidden * 2
    elif scorer == "mlp":
        score_b = slices * w.n0 * (2 * d * e + 4) + \
            w.n_kv * (2 * d * w.hidden * 2 + w.hidden * 4)
    else:
        score_b = None
    select_b = slices * (w.n0 * 8 + w.budget * 4)
    evs = stack.compress_events[1:] or stack.compress_events
    moved = [int(m.item()) for m in stack.compress_moved]
    moved = moved[1:] if len(moved) > 1 else moved
    parts = [statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3
                               for ev in evs) for i in range(3)]
    total = statistics.median(ev[0].elapsed_time(ev[3]) * 1e3 for ev in evs)
    compact_b = int(statistics.median(moved)) * 2 * (2 * d * e + 8)
    out = {"per_layer_us": round(total, 1), "score_us": round(parts[0], 1),
           "select_us": round(parts[1], 1), "compact_us": round(parts[2], 1),
           "prompt_tokens": w.n0, "batch": w.batch, "budget": w.budget,
           "layers_timed": len(evs)}
    if score_b is not None:
        tot_b = score_b + select_b + compact_b
        out.update({"bytes": tot_b, "gbps": round(tot_b / total / 1e3, 1),
                    "score_gbps": round(score_b / parts[0] / 1e3, 1),
                    "compact_gbps": round(compact_b / parts[2] / 1e3, 1)})
    out["tokens_per_s"] = round(w.batch * w.n0 / (total * 1e-6), 1)
    out["note"] = ("one-shot compression of the prompt in one layer during "
                   "set-up, median over layers 2..L (the only layer of a "
                   "one-layer workload, first launches included), HIP "
                   "events")
    return out


# ---------------------------------------------------------------------------
# Device set-up
# ---------------------------------------------------------------------------

class Stack:
    """Per-layer caches, scorer weights, step runners and input pools."""

    def __init__(self, w, seed: int, pool_steps: int, dev, decay=False,
                 scorer="mlp", stochastic=False, start_pos=None):
        import torch
        import learned_kv_cache_head_amd as kve
        import synthetic as syn
        self.w, self.dev = w, dev
        T = syn.TENSOR_IDS
        b, H, d, G = w.batch, w.n_kv, w.head_dim, w.group
        # K, V, Q and the MLP's W1 in the workload's dtype (float32 for the
        # tiny single-layer workload, bf16 otherwise)
        kd = kve.F32 if w.kv_dtype == "f32" else kve.BF16
        kt = torch.float32 if w.kv_dtype == "f32" else torch.bfloat16
        self.shape = kve.Shape(b, H, G, d, w.budget + w.evict_len, kd)
        log_gamma = None
        if decay:
            # per-KV-head decay factors spread over KVpop's range (Table 3:
            # gamma from 0.999 to 0.999999), decay step 1
            g = torch.linspace(0.999, 0.999999, H, dtype=torch.float64)
            log_gamma = torch.log(g).to(torch.float32).to(dev)
        self.policy = kve.Policy(w.budget, w.sinks, w.window, w.evict_len,
                                 log_gamma=log_gamma)
        pre_shape = kve.Shape(b, H, G, d, w.n0, kd)
        scratch = kve.CacheTensors.empty(pre_shape, dev)
        scratch_pos = torch.arange(w.n0, dtype=torch.int32, device=dev)
        keep_pre = torch.empty((b, H, w.budget), dtype=torch.int32, device=dev)
        self.ws = kve.alloc_workspace(self.shape, self.shape.capacity, dev)
        self.caches, self.scorers, self.runners = [], [], []
        self.compress_events, self.compress_moved = [], []
        keep_idx = torch.arange(w.budget, dtype=torch.int32, device=dev)
        self.k_pool, self.v_pool, self.q_pool = [], [], []
        self.h_pool, self.h_buf = [], []  # gate scorer: hidden states
        cfg = w.cfg_id
        for l in range(w.layers):
            dn = syn.device_normal
            if scorer == "mlstm":
                # KVpop Appendix E.3 shapes, P = d / 2; forget bias 3 (a
                # forget gate near 0.95), input bias 0.
                P = d // 2
                wq = dn((H, 3 * P + 2, 2 * d), seed, (cfg, l, 0, T["mlstm_w"]),
                        torch.float32, dev, scale=(2 * d) ** -0.5)
                wq[:, :2 * P] *= 2.0
                gb = torch.zeros((H, 2), dtype=torch.float32, device=dev)
                gb[:, 1] = 3.0
                a = dn((H, P), seed, (cfg, l, 0, T["mlstm_a"]), torch.float32,
                       dev, scale=P ** -0.5)
                sc = kve.Scorer.mlstm(wq.to(torch.bfloat16), a, gate_b=gb,
                                      delay=w.window)
                scratch.attach_scorer_state(pre_shape, sc)
            elif scorer == "gate":
                # Fast KVzip gate on the hidden state: linear D -> 1 per KV
                # head, sigmoid; weights N(0, 1/D).
                gw = dn((H, w.hidden), seed, (cfg, l, 0, T["gate_w"]),
                        torch.bfloat16, dev, scale=w.hidden ** -0.5)
                sc = kve.Scorer.gate(gw)
            else:
                w1 = dn((H, w.hidden, 2 * d), seed, (cfg, l, 0, T["w1"]),
                        kt, dev, scale=(2 * d) ** -0.5)
                w2 = dn((H, w.hidden), seed, (cfg, l, 0, T["w2"]),
                        torch.float32, dev, scale=w.hidden ** -0.5)
                sc = kve.Scorer.mlp(w1, w2)
            # Prompt of n0 tokens, scored and compressed to B by the library.
            scratch.k.copy_(dn((b, H, w.n0, d), seed, (cfg, l, 0, T["k0"]),
                               kt, dev))
            scratch.v.copy_(dn((b, H, w.n0, d), seed, (cfg, l, 0, T["v0"]),
                               kt, dev))
            scratch.pos.copy_(scratch_pos.expand(b, H, w.n0))
            # The one-shot compression of the prompt (score every prompt
            # token, select, compact), timed per layer with events.
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            if scorer == "gate":
                hid0 = dn((b, w.n0, w.hidden), seed, (cfg, l, 0, T["hidden0"]),
                          torch.bfloat16, dev)
                ev[0].record()
                kve.kve_score(pre_shape, sc, scratch, 0, w.n0, hidden=hid0)
                ev[1].record()
                del hid0
            else:
                ev[0].record()
                kve.kve_score(pre_shape, sc, scratch, 0, w.n0)
                ev[1].record()
            kve.kve_select_evict(pre_shape, self.policy, scratch, w.n0,
                                 w.budget, keep_pre)
            ev[2].record()
            kve.kve_compact(pre_shape, scratch, w.n0, keep_pre, w.budget)
            ev[3].record()
            self.compress_events.append(ev)
            self.compress_moved.append((keep_pre != keep_idx).sum())
            c = kve.CacheTensors.empty(self.shape, dev)
            B = w.budget
            c.k[:, :, :B].copy_(scratch.k[:, :, :B])
            c.v[:, :, :B].copy_(scratch.v[:, :, :B])
            c.score[:, :, :B].copy_(scratch.score[:, :, :B])
            c.pos[:, :, :B].copy_(scratch.pos[:, :, :B])
            # The recurrent state does not depend on the capacity.
            c.scorer_state = scratch.scorer_state
            scratch.scorer_state = None
            # Decoding continues at position start_pos (default: right after
            # the prompt); the compressed cache is the same either way.
            st = kve.DecodeState(B, B, w.n0 if start_pos is None else start_pos)
            self.caches.append(c)
            self.scorers.append(sc)
            pol = self.policy
            if stochastic:
                # ForesightKV's stochastic eviction: standard Gumbel noise
                # per slot, drawn once per layer (resident input).
                u = torch.rand((b, H, self.shape.capacity), generator=torch.Generator(
                    device=dev).manual_seed(seed * 1000 + l), device=dev)
                gum = -torch.log(-torch.log(u.clamp_(1e-7, 1 - 1e-7)))
                pol = kve.Policy(w.budget, w.sinks, w.window, w.evict_len,
                                 log_gamma=self.policy.log_gamma, gumbel=gum)
            self.runners.append(kve.LayerStep(self.shape, pol, sc, c, st,
                                              self.ws))
            self.k_pool.append(dn((pool_steps, b, H, d), seed,
                                  (cfg, l, 1, T["k_new"]), kt, dev))
            self.v_pool.append(dn((pool_steps, b, H, d), seed,
                                  (cfg, l, 1, T["v_new"]), kt, dev))
            self.q_pool.append(dn((pool_steps, b, H * G, d), seed,
                                  (cfg, l, 1, T["q"]), kt, dev))
            if scorer == "gate":
                self.h_pool.append(dn((pool_steps, b, w.hidden), seed,
                                      (cfg, l, 1, T["hidden_new"]),
                                      torch.bfloat16, dev))
                self.h_buf.append(torch.zeros((b, w.evict_len, w.hidden),
                                              dtype=torch.bfloat16, device=dev))
        del scratch
        self.pool_steps = pool_steps
        self.out = torch.empty((b, H * G, d), dtype=torch.float32, device=dev)
        self.keep_scratch = [torch.empty((b, H, self.shape.capacity),
                                         dtype=torch.int32, device=dev)
                             for _ in range(w.layers)]
        torch.cuda.synchronize()

    def run_step(self, i: int, keep_for=None):
        """Decode step i over all layers. keep_for(l) may supply the buffer
        that receives the kept slots of an evicting call."""
        j = i % self.pool_steps
        for l, r in enumerate(self.runners):
            keep = self.keep_scratch[l]
            if keep_for is not None and r.evicts_next():
                keep = keep_for(l)
            if self.h_pool:
                r(self.k_pool[l][j], self.v_pool[l][j], self.q_pool[l][j],
                  self.out, None, keep, hidden_new=self.h_pool[l][j],
                  hidden_buf=self.h_buf[l])
            else:
                r(self.k_pool[l][j], self.v_pool[l][j], self.q_pool[l][j],
                  self.out, None, keep)


# ---------------------------------------------------------------------------
# Oracle CPU baseline (bounded sample)
# ---------------------------------------------------------------------------

def cpu_baseline(w, seed: int, sample_batch: int, sample_steps: int,
                 scorer: str = "mlp") -> dict:
    """Time the float64 oracle on one layer of the same workload for
    ``sample_batch`` sequences over ``sample_steps`` decode steps (whole
    eviction cycles), starting from its own compressed prompt; scale to the
    full stack's tokens/s (tokens / (time x layers))."""
    import numpy as np
    import oracle as O
    import synthetic as syn
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    if scorer == "mlstm":
        return cpu_baseline_mlstm(w, seed, sample_batch, sample_steps, threads)
    if scorer == "gate":
        return cpu_baseline_gate(w, seed, sample_steps, threads)
    ws = syn.workload(w.cfg_id, batch=sample_batch)
    ctx = syn.initial_context(ws, seed, 0)
    wts = syn.draw_mlp_weights(ws, seed, 0)

    def scores(k64, v64):
        out = np.empty(k64.shape[:3], dtype=np.float32)
        for bi in range(k64.shape[0]):
            for h in range(k64.shape[1]):
                out[bi, h] = O.score_to_f32(O.mlp_score(
                    k64[bi, h], v64[bi, h], wts["w1"].f64[h], wts["b1"].f64[h],
                    wts["w2"].f64[h], wts["b2"].f64[h], ws.act))
        return out

    lay = O.OracleLayer(ctx["k0"].f64, ctx["v0"].f64,
                        scores(ctx["k0"].f64, ctx["v0"].f64),
                        O.Policy(ws.budget, ws.sinks, ws.window, ws.evict_len),
                        ws.group)
    lay.prefill_compress()
    del ctx
    inputs = [syn.step_inputs(ws, seed, 0, i) for i in range(sample_steps)]
    t0 = time.perf_counter()
    for x in inputs:
        sn = scores(x["k_new"].f64[:, :, None], x["v_new"].f64[:, :, None])
        lay.step(x["k_new"].f64, x["v_new"].f64, sn[:, :, 0], x["q"].f64)
    dt = time.perf_counter() - t0
    tokens = sample_batch * sample_steps
    return {
        "value": tokens / (dt * w.layers),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle, 1 of {w.layers} layers, {sample_batch} "
                   f"of {w.batch} sequences, {sample_steps} decode steps "
                   f"({sample_steps // w.evict_len} eviction cycles) from a "
                   f"compressed {w.n0}-token prompt; {dt:.1f} s wall; scaled "
                   f"to the {w.layers}-layer step as tokens/(time x layers)"),
    }


def cpu_baseline_gate(w, seed, sample_steps, threads) -> dict:
    """The oracle's decode loop with the hidden-state gate, one layer of the
    batch-1 stack, from a random cache of B entries (the prompt's one-shot
    compression is not timed and not run: its product is a cache of B)."""
    import numpy as np
    import oracle as O
    import synthetic as syn
    ws = syn.workload(w.cfg_id, batch=1, n0=w.budget)
    ctx = syn.initial_context(ws, seed, 0)
    gw = syn.draw_gate_weights(ws, seed, 0)

    def scores(hid64):
        return np.stack([np.stack([O.score_to_f32(O.gate_score(
            hid64[bi], gw["w"].f64[h], gw["b"].f64[h]))
            for h in range(ws.n_kv)]) for bi in range(hid64.shape[0])])

    s0 = scores(ctx["hidden0"].f64)
    lay = O.OracleLayer(ctx["k0"].f64, ctx["v0"].f64, s0,
                        O.Policy(ws.budget, ws.sinks, ws.window, ws.evict_len),
                        ws.group)
    del ctx
    inputs = [syn.step_inputs(ws, seed, 0, i) for i in range(sample_steps)]
    t0 = time.perf_counter()
    for x in inputs:
        sn = scores(x["hidden_new"].f64[:, None])[:, :, 0]
        lay.step(x["k_new"].f64, x["v_new"].f64, sn, x["q"].f64)
    dt = time.perf_counter() - t0
    return {
        "value": sample_steps / (dt * w.layers),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle with the hidden-state gate, 1 of "
                   f"{w.layers} layers, batch 1, {sample_steps} decode steps "
                   f"({sample_steps // w.evict_len} eviction cycles) from a "
                   f"random cache of B = {w.budget} entries; {dt:.1f} s wall; "
                   f"scaled to the {w.layers}-layer step as "
                   f"tokens/(time x layers)"),
    }


def cpu_baseline_mlstm(w, seed, sample_batch, sample_steps, threads) -> dict:
    """The oracle's decode loop with the stateful scorer: every new token
    is absorbed by the slice's float64 recurrence and the token leaving the
    window is scored (the prompt is absorbed untimed)."""
    import numpy as np
    import oracle as O
    import synthetic as syn
    ws = syn.workload(w.cfg_id, batch=sample_batch, scorer="mlstm",
                      hidden=w.head_dim // 2)
    ctx = syn.initial_context(ws, seed, 0)
    wts = syn.draw_mlstm_weights(ws, seed, 0)
    P = w.head_dim // 2

    def head(h):
        x, gb = wts["w"].f64[h], wts["gate_b"].f64[h]
        return O.MlstmWeights(x[:P], x[P:2 * P], x[2 * P:3 * P], x[3 * P],
                              x[3 * P + 1], gb[0], gb[1], wts["a"].f64[h],
                              float(wts["b"].f64[h]))
    W = ws.window
    scs = [[O.MlstmScorer(head(h), W) for h in range(ws.n_kv)]
           for _ in range(sample_batch)]
    s0 = np.zeros((sample_batch, ws.n_kv, ws.n0), np.float32)
    for bi in range(sample_batch):
        for h in range(ws.n_kv):
            for t in range(ws.n0):
                r = scs[bi][h].push(np.concatenate(
                    [ctx["k0"].f64[bi, h, t], ctx["v0"].f64[bi, h, t]]))
                if r is not None:
                    s0[bi, h, r[0]] = r[1]
    lay = O.OracleLayer(ctx["k0"].f64, ctx["v0"].f64, s0,
                        O.Policy(ws.budget, ws.sinks, ws.window, ws.evict_len),
                        ws.group)
    lay.prefill_compress()
    del ctx
    inputs = [syn.step_inputs(ws, seed, 0, i) for i in range(sample_steps)]
    t0 = time.perf_counter()
    for i, x in enumerate(inputs):
        su = np.empty((sample_batch, ws.n_kv), np.float32)
        for bi in range(sample_batch):
            for h in range(ws.n_kv):
                _, su[bi, h] = scs[bi][h].push(np.concatenate(
                    [x["k_new"].f64[bi, h], x["v_new"].f64[bi, h]]))
        lay.append(x["k_new"].f64, x["v_new"].f64,
                   np.zeros((sample_batch, ws.n_kv), np.float32))
        lay.set_scores(ws.n0 + i - W, su)
        lay.maybe_evict()
        lay.attend(x["q"].f64)
    dt = time.perf_counter() - t0
    tokens = sample_batch * sample_steps
    return {
        "value": tokens / (dt * w.layers),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle with the mLSTM scorer, 1 of {w.layers} "
                   f"layers, {sample_batch} of {w.batch} sequences, "
                   f"{sample_steps} decode steps from a compressed "
                   f"{w.n0}-token prompt (absorbed untimed); {dt:.1f} s wall; "
                   f"scaled to the {w.layers}-layer step as "
                   f"tokens/(time x layers)"),
    }


# ---------------------------------------------------------------------------
# Prefill: running top-k selection and Eq. 26 masked prefill attention
# ---------------------------------------------------------------------------

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def prefill_kept_pairs(n: int, budget: int) -> int:
    """(query, key) pairs the Eq. 26 mask keeps for an n-token prompt: every
    causal pair while q + 1 <= B, then B per query."""
    return sum(min(q + 1, budget) for q in range(n))


def run_prefill(args, w, dev) -> dict:
    """Time one layer's prefill: kve_prefill_select (ranks, cutoffs) and
    kve_prefill_attn over the workload's prompt for the whole batch, with
    the library's scores (the MLP over [k; v], or for the Qwen2.5-14B
    workload the hidden-state gate over the prompt's hidden states)."""
    import torch
    import learned_kv_cache_head_amd as kve
    import synthetic as syn
    T = syn.TENSOR_IDS
    b, H, G, d, n = w.batch, w.n_kv, w.group, w.head_dim, w.n0
    cfg, l, seed = w.cfg_id, 0, args.seed
    shape = kve.Shape(b, H, G, d, n, kve.BF16)
    pol = kve.Policy(w.budget, w.sinks, w.window, w.evict_len)
    dn = syn.device_normal
    c = kve.CacheTensors.empty(shape, dev)
    c.k.copy_(dn((b, H, n, d), seed, (cfg, l, 0, T["k0"]), torch.bfloat16, dev))
    c.v.copy_(dn((b, H, n, d), seed, (cfg, l, 0, T["v0"]), torch.bfloat16, dev))
    c.pos.copy_(torch.arange(n, dtype=torch.int32, device=dev).expand(b, H, n))
    if w.scorer == "gate":
        gw = dn((H, w.hidden), seed, (cfg, l, 0, T["gate_w"]), torch.bfloat16,
                dev, scale=w.hidden ** -0.5)
        hid0 = dn((b, n, w.hidden), seed, (cfg, l, 0, T["hidden0"]),
                  torch.bfloat16, dev)
        kve.kve_score(shape, kve.Scorer.gate(gw), c, 0, n, hidden=hid0)
        del hid0
    elif w.scorer == "mlp":
        w1 = dn((H, w.hidden, 2 * d), seed, (cfg, l, 0, T["w1"]),
                torch.bfloat16, dev, scale=(2 * d) ** -0.5)
        w2 = dn((H, w.hidden), seed, (cfg, l, 0, T["w2"]), torch.float32, dev,
                scale=w.hidden ** -0.5)
        kve.kve_score(shape, kve.Scorer.mlp(w1, w2), c, 0, n)
    else:
        raise ValueError(f"--prefill takes an MLP or gate workload, not "
                         f"{w.scorer}")
    q = dn((b, H * G, n, d), seed, (cfg, l, 2, T["q"]), torch.bfloat16, dev)
    rank = torch.empty((b, H, n), dtype=torch.int32, device=dev)
    tau = torch.empty_like(rank)
    out = torch.empty((b, H * G, n, d), dtype=torch.float32, device=dev)
    lse = torch.empty((b, H * G, n), dtype=torch.float32, device=dev)
    ws = torch.empty(kve.kve_prefill_workspace_bytes(shape, n) // 8,
                     dtype=torch.int64, device=dev)
    wsa = torch.empty(kve.kve_prefill_attn_workspace_bytes(shape, pol, n) // 4,
                      dtype=torch.int32, device=dev)
    steps = args.steps if args.steps is not None else 3
    warmup = args.warmup if args.warmup is not None else 1
    for _ in range(warmup):
        kve.kve_prefill_select(shape, pol, c, n, rank, tau, ws)
        kve.kve_prefill_attn(shape, pol, c, n, rank, tau, q, out, lse, wsa)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        kve.kve_prefill_select(shape, pol, c, n, rank, tau, ws)
        ev[2 * i + 1].record()
        kve.kve_prefill_attn(shape, pol, c, n, rank, tau, q, out, lse, wsa)
        ev[2 * i + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
    attn_ms = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2])
                  for i in range(steps)) / steps
    kept = prefill_kept_pairs(n, w.budget)
    flops = kept * 4 * d * H * G * b  # q.k and p.v over the kept pairs
    causal = n * (n + 1) // 2
    achieved = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": ("prefill tokens/s of one layer: running top-k selection "
                   "(KVpop Eq. 26) + masked prefill attention"),
        "value": round(b * n * steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall * 1e3 / steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload + "-prefill-1layer", "batch": b,
                   "prompt_len": n, "n_kv_heads": H, "n_q_heads": H * G,
                   "head_dim": d, "budget": w.budget, "sinks": w.sinks,
                   "window": w.window, "scorer": w.scorer, "parallelism": "none"},
        "select_ms": round(sel_ms, 3),
        "attn_ms": round(attn_ms, 3),
        "mask_density": round(kept / causal, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "kernel": "key lists + prefill_attn_kernel (Eq. 26 masked attention)",
                     "algorithmic_flops_per_launch": int(flops),
                     "mean_launch_ms": round(attn_ms, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(w, seed)
    return result


def cpu_baseline_prefill(w, seed) -> dict:
    """The oracle's prefill (ranks, cutoffs, Eq. 26 mask, float64 masked
    attention) for one sequence and one KV head of the same prompt; scaled
    to tokens/s of the layer as n / (time x KV heads)."""
    import numpy as np
    import oracle as O
    import synthetic as syn
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    # The oracle's mask is n x n: prompts longer than 8192 tokens are
    # sampled by their first 8192, and the time is scaled by kept pairs.
    n_full, d, G = w.n0, w.head_dim, w.group
    n = min(n_full, 8192)
    rng = syn.rng_for(seed, w.cfg_id, 0, -1, "misc")
    K = rng.standard_normal((1, n, d))
    V = rng.standard_normal((1, n, d))
    Q = rng.standard_normal((G, n, d))
    s = rng.standard_normal(n).astype(np.float32)
    t0 = time.perf_counter()
    r = O.prefill_ranks(s)
    tau = O.prefill_cutoffs(r, w.sinks, w.window, w.budget - w.sinks - w.window)
    M = O.prefill_mask(r, tau, w.sinks, w.window)[None]
    O.prefill_attention(Q, K, V, M, G)
    dt = time.perf_counter() - t0
    scale = prefill_kept_pairs(n_full, w.budget) / prefill_kept_pairs(n, w.budget)
    part = (f"the first {n} of {n_full} tokens of one sequence"
            if n < n_full else f"one {n}-token sequence")
    return {"value": round(n_full / (dt * scale * w.n_kv), 3),
            "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"float64 oracle prefill (ranks, cutoffs, mask, masked "
                       f"attention) of {part} and one of {w.n_kv} KV heads "
                       f"({G} query heads); {dt:.1f} s wall; scaled to the "
                       f"layer as n / (time x KV heads"
                       + (f" x {scale:.1f}, the ratio of kept pairs)"
                          if n < n_full else ")"))}


# ---------------------------------------------------------------------------
# Prefill scoring with the low-rank sink-attention gate
# ---------------------------------------------------------------------------

SINK_GATE_WORKLOAD = 5  # Qwen2.5-14B layer, 131072-token prompt
SINK_GATE_RANK = 16     # D' = S = 16 (Fast KVzip section 3.4)
SINK_GATE_WORKLOAD_NAME = "qwen2.5-14b-1layer-131k-sink-gate"


def sink_gate_flops(n: int, D: int, H: int, G: int) -> int:
    """MFMA work of the gate over n hidden states: the W_k and W_q
    projections, 2 n D (H + H G) D' flops (the normalisations, logits and
    softmax are O(n H G D') and not counted)."""
    return 2 * n * D * H * (1 + G) * SINK_GATE_RANK


def sink_gate_bytes(n: int, D: int, H: int, G: int) -> int:
    """Algorithmic HBM bytes: the n bf16 hidden states read once, the bf16
    projection weights once, one float32 score per (token, KV head)."""
    return n * D * 2 + H * (1 + G) * SINK_GATE_RANK * D * 2 + n * H * 4


def run_sink_gate(args, dev) -> dict:
    """Time one layer's gate scoring of a whole prompt (kve_score with the
    sink-attention gate over all n hidden states)."""
    import torch
    import learned_kv_cache_head_amd as kve
    import synthetic as syn
    T = syn.TENSOR_IDS
    w = syn.workload(SINK_GATE_WORKLOAD, scorer="sink_gate")
    b, H, G, D, n = w.batch, w.n_kv, w.group, w.hidden, w.n0
    cfg, l, seed = w.cfg_id, 0, args.seed
    dn = syn.device_normal
    shape = kve.Shape(b, H, G, w.head_dim, n, kve.BF16)
    cache = kve.CacheTensors.empty(shape, dev)
    hidden = dn((b, n, D), seed, (cfg, l, 0, T["hidden0"]), torch.bfloat16, dev)
    wt = dn((H * (1 + G) * SINK_GATE_RANK, D), seed, (cfg, l, 0, T["sg_w"]),
            torch.bfloat16, dev, scale=D ** -0.5)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    norm = 0.5 + torch.rand(32, generator=gen, device=dev)
    sinks = torch.randn((SINK_GATE_RANK, SINK_GATE_RANK), generator=gen,
                        device=dev)
    bias = torch.rand(H * G, generator=gen, device=dev)
    sc = kve.Scorer.sink_gate(wt, sinks, norm=norm, b=bias)
    steps = args.steps if args.steps is not None else 20
    warmup = args.warmup if args.warmup is not None else 3
    for _ in range(warmup):
        kve.kve_score(shape, sc, cache, 0, n, hidden=hidden)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        kve.kve_score(shape, sc, cache, 0, n, hidden=hidden)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps
    if args.calib_copy:
        calib_copy(dev)
    flops = sink_gate_flops(b * n, D, H, G)
    nbytes = sink_gate_bytes(b * n, D, H, G)
    achieved = flops / (ms * 1e-3) / 1e12
    ratio = recorded_ratio(f"sink_gate_{SINK_GATE_WORKLOAD_NAME}.txt",
                           SCORE_SOURCE, "score_source_sha256")
    result = {
        "metric": ("prefill gate tokens/s of one layer: low-rank "
                   "sink-attention gate scores of every prompt token"),
        "value": round(b * n * steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": SINK_GATE_WORKLOAD_NAME,
                   "batch": b, "prompt_len": n, "hidden_dim": D,
                   "n_kv_heads": H, "n_q_heads": H * G,
                   "gate_rank": SINK_GATE_RANK, "n_sink": SINK_GATE_RANK,
                   "parallelism": "none"},
        "hbm_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if ratio is None else int(ratio * nbytes),
                     "kernel": "sink_gate_kernel (projections + gate)",
                     "algorithmic_flops_per_launch": int(flops),
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "mean_launch_ms": round(ms, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_sink_gate(w, seed)
    return result


def cpu_baseline_sink_gate(w, seed, sample: int = 8192) -> dict:
    """The oracle's gate on ``sample`` tokens of the same layer shape, scaled
    to tokens/s."""
    import numpy as np
    import oracle as O
    import synthetic as syn
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    H, G, D = w.n_kv, w.group, w.hidden
    wts = syn.draw_sink_gate_weights(w, seed, 0)
    wt = wts["w"].f64
    ow = O.SinkGateWeights(wt[:H * 16].reshape(H, 16, D),
                           wt[H * 16:].reshape(H, G, 16, D),
                           wts["norm"].f64[:16], wts["norm"].f64[16:],
                           wts["sinks"].f64, wts["b"].f64.reshape(H, G))
    rng = syn.rng_for(seed, w.cfg_id, 0, -1, "hidden0")
    x = syn.Stored(rng.standard_normal((sample, D)).astype(np.float32),
                   "bf16").f64
    t0 = time.perf_counter()
    O.sink_gate_score(x, ow)
    dt = time.perf_counter() - t0
    return {"value": round(sample / dt, 1), "unit": "tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"float64 oracle gate over {sample} of {w.n0} prompt "
                       f"tokens of one layer (D = {D}, {H} KV heads, "
                       f"{H * G} query heads); {dt:.1f} s wall")}


# ---------------------------------------------------------------------------
# Recorded rocprofv3 traffic of the attention kernel
# ---------------------------------------------------------------------------

def recorded_ratio(profile: str, source: str, sha_key: str):
    """Measured HBM bytes over algorithmic bytes of one launch, from a
    committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE passes,
    each scaled by what the counter reads for a plain copy of known size), or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    src = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if rec.get(sha_key) != src:
        return None
    try:
        return float(rec["traffic_over_algorithmic"])
    except (KeyError, ValueError):
        return None


def traffic_ratio(workload: str):
    """Recorded traffic ratio of the decode attention kernel."""
    return recorded_ratio(f"decode_attn_{workload}_traffic.txt", ATTN_SOURCE,
                          "attention_source_sha256")


# ---------------------------------------------------------------------------
# Timing over eviction cycles
# ---------------------------------------------------------------------------

def preroll_steps(L: int, warmup: int, steps: int) -> int:
    """Untimed decode steps that set-up runs after the prompt compression
    (which leaves B entries; the t-th step after it evicts when t is a
    multiple of L) so that timed step steps // 2 is an evicting step."""
    e = steps // 2
    return (-(warmup + 1 + e)) % L


def window_has_eviction(L: int, preroll: int, warmup: int, steps: int) -> bool:
    """Whether the timed steps (the t-th decode step after the prompt
    compression evicts when t is a multiple of L) include an evicting one."""
    first = preroll + warmup + 1
    last = preroll + warmup + steps
    return last // L > (first - 1) // L


def cycle_profile(step_ms, evicts, L: int, batch: int, pos0: int,
                  max_points: int = 8):
    """Throughput of whole eviction cycles inside the window (L consecutive
    steps that end with an evicting step), at up to ``max_points`` cycles
    spread evenly over it: the decoded position of each cycle's first token
    and batch * L / (sum of its step times)."""
    ends = [i for i, e in enumerate(evicts) if e and i + 1 >= L]
    cycles = [(i + 1 - L, sum(step_ms[i + 1 - L:i + 1])) for i in ends]
    if not cycles:
        return []
    if len(cycles) > max_points:
        pick = [round(j * (len(cycles) - 1) / (max_points - 1))
                for j in range(max_points)]
        cycles = [cycles[j] for j in pick]
    return [{"start_pos": pos0 + s0,
             "tokens_per_s": round(batch * L / (ms * 1e-3), 1)}
            for s0, ms in cycles]


def attn_rows(w, n: int, evicts: bool) -> int:
    """Rows the attention of a step reads: B after an eviction, else the
    count after the append."""
    return w.budget if evicts else n


def cycle_fold(step_ms, evicts, L: int) -> float:
    """Time of one eviction cycle (L decode steps, one of them evicting)
    from per-step times of a window: the mean evicting step plus L - 1 mean
    non-evicting steps. Over whole cycles this is the window's time per
    cycle; a shorter window centred on an eviction weighs that step as one
    step in L instead of one in the window."""
    ev = [t for t, e in zip(step_ms, evicts) if e]
    ne = [t for t, e in zip(step_ms, evicts) if not e]
    if not ev:
        raise ValueError("the timed window holds no evicting step")
    t = sum(ev) / len(ev)
    if L > 1:
        if not ne:
            raise ValueError("the timed window holds no non-evicting step")
        t += (L - 1) * sum(ne) / len(ne)
    return t


def cycle_bytes(w, lens, moved, scorer: str) -> int:
    """Algorithmic bytes of one eviction cycle over all layers: the L - 1
    non-evicting steps at B + 1 .. B + L - 1 rows (fused append), plus the
    evicting step (append, scorer, select, compaction of the rows the timed
    evictions moved on average, attention over B rows)."""
    B, L = w.budget, w.evict_len
    per_layer = sum(attn_launch_bytes(w, n, True) for n in range(B + 1, B + L))
    mv = list(moved.values())
    mean_moved = sum(mv) / len(mv) if mv else 0
    per_layer += evict_extra_bytes(w, B + L, int(round(mean_moved)), scorer)
    per_layer += attn_launch_bytes(w, B, False)
    return per_layer * w.layers


def timing_note(events: bool, flushed: bool, flush_mb: int, L: int,
                wall: float, wall_tokens_s: float) -> dict:
    if not events:
        return {"method": "wall clock over the timed steps"}
    how = ("per-step HIP events on the launch stream, folded into one "
           f"eviction cycle: mean evicting step + {L - 1} x mean "
           "non-evicting step")
    if flushed:
        how += (f"; a {flush_mb} MB copy before every step, outside the "
                "timed spans, keeps the cache out of the Infinity Cache")
    return {"method": how, "wall_ms": round(wall * 1e3, 3),
            "wall_tokens_per_s": round(wall_tokens_s, 1)}


# ---------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default 4 eviction cycles)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 1 eviction cycle)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(WORKLOAD_BY_NAME))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time only the whole region (no per-launch events)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decay", action="store_true",
                    help="rank with KVpop temporal decay (static priority)")
    ap.add_argument("--start-pos", type=int, default=None,
                    help="position of the first decoded token (default: the "
                         "prompt length); the cache is the prompt compressed "
                         "to B, relabelled as a cache at that position")
    ap.add_argument("--stochastic", action="store_true",
                    help="ForesightKV stochastic eviction (Gumbel noise per "
                         "slot in the policy)")
    ap.add_argument("--scorer", default="mlp", choices=["mlp", "mlstm"],
                    help="stateless MLP over [k; v], or the stateful mLSTM "
                         "scorer with delayed read-out")
    ap.add_argument("--cpu-batch", type=int, default=None,
                    help="oracle sample sequences (default 16; 2 for mLSTM)")
    ap.add_argument("--cpu-steps", type=int, default=None)
    ap.add_argument("--prefill", action="store_true",
                    help="time one layer's prefill (running top-k selection "
                         "and Eq. 26 masked attention) instead of decode")
    ap.add_argument("--sink-gate", action="store_true",
                    help="time one layer's prompt scoring with the low-rank "
                         "sink-attention gate (Qwen2.5-14B, 131072 tokens) "
                         "instead of decode")
    ap.add_argument("--hw-reference", action="store_true",
                    help="print reference measurements instead of a bench "
                         "line: the MFMA / vector-ALU issue probe and the "
                         "vendor libraries' GEMM and fused attention at the "
                         "sink-gate and prefill shapes")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="copy this many MB before every timed step (not "
                         "timed) so the cache is read from HBM, not the "
                         "Infinity Cache; steps are timed alone by events")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed region, run a plain 1 GiB "
                         "elementwise copy (counter calibration)")
    ap.add_argument("--preroll", type=int, default=None,
                    help="untimed decode steps after the prompt compression "
                         "(default: the count that puts an eviction at timed "
                         "step steps // 2). 0 decodes from the prompt's end "
                         "(e.g. 8K to 32K in 24576 steps); with "
                         "--no-kernel-events a counter pass may also stay "
                         "clear of evictions")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "libkvevict runs on one GPU; --gpus "
                          f"{args.gpus} is not supported (the step shards "
                          "by batch or KV head with no exchange, but only "
                          "the one-GPU path is built)"}))
        return 2
    if args.flush_mb > 0 and args.no_kernel_events:
        print(json.dumps({"error": "--flush-mb times every step with events; "
                          "it cannot be combined with --no-kernel-events"}))
        return 2
    if args.preroll is not None and not (args.sink_gate or args.prefill):
        w0 = workload_for(args.workload)
        L0 = w0.evict_len
        st0 = args.steps if args.steps is not None else max(4 * L0, 64)
        wu0 = args.warmup if args.warmup is not None else max(L0, 8)
        if args.preroll < 0 or not (args.no_kernel_events or
                                    window_has_eviction(L0, args.preroll,
                                                        wu0, st0)):
            print(json.dumps({"error": "--preroll takes a count >= 0, and "
                              "without --no-kernel-events the timed window "
                              "must still hold an evicting step (the "
                              "per-step fold needs one)"}))
            return 2

    import torch
    import synthetic as syn
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.hw_reference:
        log("hardware references: issue probe, vendor GEMM and attention")
        print(json.dumps({"issue_probe": issue_probe(dev),
                          "library_reference": library_reference(dev)}),
              flush=True)
        return 0
    if args.sink_gate:
        log("sink gate: qwen2.5-14b layer, 131072-token prompt")
        print(json.dumps(run_sink_gate(args, dev)), flush=True)
        return 0
    w = workload_for(args.workload)
    if args.prefill:
        log(f"prefill {args.workload}: batch={w.batch} prompt={w.n0} B={w.budget}")
        print(json.dumps(run_prefill(args, w, dev)), flush=True)
        return 0
    L = w.evict_len
    # four eviction cycles after one, at least 64 steps (the tiny workload
    # evicts one entry every step)
    steps = args.steps if args.steps is not None else max(4 * L, 64)
    warmup = args.warmup if args.warmup is not None else max(L, 8)
    if steps < 1 or warmup < 0:
        print(json.dumps({"error": "--steps must be at least 1 and --warmup "
                          "at least 0"}))
        return 2
    # The cache holds B entries after set-up and evicts on every L-th step.
    # Set-up advances it by `preroll` untimed decode steps so that an
    # eviction falls in the middle of the timed window, whatever --steps is.
    preroll = (preroll_steps(L, warmup, steps) if args.preroll is None
               else args.preroll)
    pool = min(preroll + warmup + steps, 3 * L)
    log(f"workload {args.workload}: layers={w.layers} batch={w.batch} "
        f"B={w.budget} L={L} steps={steps} warmup={warmup}")
    t0 = time.perf_counter()
    scorer = "gate" if w.scorer == "gate" else args.scorer
    if args.start_pos is not None and args.start_pos < w.n0:
        print(json.dumps({"error": "--start-pos must be at least the prompt "
                          f"length {w.n0}"}))
        return 2
    stack = Stack(w, args.seed, pool, dev, decay=args.decay,
                  scorer=scorer, stochastic=args.stochastic,
                  start_pos=args.start_pos)
    for i in range(preroll):
        stack.run_step(i)
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t0:.1f} s (cache advanced by "
        f"{preroll} decode steps to the phase the timed window starts at)")

    for i in range(warmup):
        stack.run_step(preroll + i)
    torch.cuda.synchronize()
    log("warm-up done")

    # Expected retained count per step, and keep buffers of the evictions
    # inside the timed region (to count the rows that compaction moves).
    n_layers = w.layers
    lens = []
    keep_bufs = {}
    n = stack.runners[0].state.len
    for i in range(steps):
        n += 1
        ev = n >= w.budget + L
        lens.append((n, ev))
        if ev:
            n = w.budget

    taken = {}

    def keep_for(l):
        c = taken.get(l, 0)
        taken[l] = c + 1
        buf = torch.empty((w.batch, w.n_kv, w.budget), dtype=torch.int32,
                          device=dev)
        keep_bufs[(l, c)] = buf
        return buf

    # One event after every step (plus one before the first): a step without
    # an eviction is exactly one attention launch per layer, so its duration
    # over the layer count is the mean launch duration of the kernel,
    # measured on the stream the launches go to. The per-step times also
    # fold the window into one eviction cycle (cycle_fold).
    use_events = not args.no_kernel_events
    events = None
    if use_events:
        events = [torch.cuda.Event(enable_timing=True)
                  for _ in range(steps + 1)]
    # --flush-mb: a plain copy of that many bytes before every step pushes the
    # cache out of the Infinity Cache (a single layer at batch 16 fits in
    # it); each step is then timed alone with events and the flush excluded.
    flush = None
    if args.flush_mb > 0:
        nb = args.flush_mb * (1 << 20) // 2
        flush = (torch.ones(nb, dtype=torch.uint8, device=dev),
                 torch.empty(nb, dtype=torch.uint8, device=dev))
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if use_events:
        events[0].record()
    for s in range(steps):
        if flush is not None:
            flush[1].copy_(flush[0])
            starts[s].record()
        stack.run_step(preroll + warmup + s, keep_for)
        if use_events:
            events[s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {steps} steps in {wall * 1e3:.1f} ms")
    step_ms_list = None
    if flush is not None:
        step_ms_list = [starts[s].elapsed_time(events[s + 1])
                        for s in range(steps)]
        wall = sum(step_ms_list) * 1e-3
        log(f"steps alone (flush excluded): {wall * 1e3:.1f} ms")

    if args.calib_copy:
        calib_copy(dev)

    # Algorithmic bytes over the timed region.
    moved = {}
    for (l, c), buf in keep_bufs.items():
        idx = torch.arange(w.budget, dtype=torch.int32, device=dev)
        moved[(l, c)] = int((buf != idx).sum().item())
    total_bytes = 0
    attn_bytes, attn_ms = [], []
    ev_count = {}
    for s, (n, ev) in enumerate(lens):
        for l in range(n_layers):
            if ev:
                c = ev_count.get(l, 0)
                ev_count[l] = c + 1
                total_bytes += evict_extra_bytes(w, n, moved[(l, c)],
                                                 scorer)
                total_bytes += attn_launch_bytes(w, w.budget, False)
            else:
                total_bytes += attn_launch_bytes(w, n, True)
        if use_events and not ev:
            step_ms = (step_ms_list[s] if step_ms_list is not None
                       else events[s].elapsed_time(events[s + 1]))
            attn_bytes += [attn_launch_bytes(w, n, True)] * n_layers
            attn_ms += [step_ms / n_layers] * n_layers

    n_evict = sum(1 for _, ev in lens if ev)
    log(f"timed window: {n_evict} evicting step(s) of {steps}, attention "
        f"over {sum(attn_rows(w, n, ev) for n, ev in lens) / steps:.1f} "
        f"rows on average (cycle mean {w.budget + (L - 1) / 2:.1f})")
    wall_tokens_s = w.batch * steps / wall
    if use_events:
        step_ms_all = (step_ms_list if step_ms_list is not None else
                       [events[s].elapsed_time(events[s + 1])
                        for s in range(steps)])
        cyc_ms = cycle_fold(step_ms_all, [ev for _, ev in lens], L)
        cyc_bytes = cycle_bytes(w, lens, moved, scorer)
        tokens_s = w.batch * L / (cyc_ms * 1e-3)
        ms_step = cyc_ms / L
        step_gbps = cyc_bytes / (cyc_ms * 1e-3) / 1e9
    else:
        tokens_s = wall_tokens_s
        ms_step = wall * 1e3 / steps
        step_gbps = total_bytes / wall / 1e9
    roof = None
    if use_events and attn_ms:
        mean_ms = sum(attn_ms) / len(attn_ms)
        mean_bytes = sum(attn_bytes) / len(attn_bytes)
        achieved = mean_bytes / (mean_ms * 1e-3) / 1e9
        ratio = traffic_ratio(args.workload)
        traffic = None if ratio is None else int(ratio * mean_bytes)
        roof = {"bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "attn_kernel (decode attention, fused append)",
                "launches": len(attn_ms),
                "mean_launch_us": round(mean_ms * 1e3, 2),
                "algorithmic_bytes_per_launch": int(mean_bytes)}
    result = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.kv_dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": w.layers,
                   "batch": w.batch, "n_kv_heads": w.n_kv,
                   "n_q_heads": w.n_q, "head_dim": w.head_dim,
                   "budget": w.budget, "sinks": w.sinks, "window": w.window,
                   "evict_len": w.evict_len, "prompt_len": w.n0,
                   "start_pos": (w.n0 if args.start_pos is None
                                 else args.start_pos),
                   "scorer": (f"mlp {2 * w.head_dim}-{w.hidden}-1 relu"
                              if scorer == "mlp" else
                              f"gate {w.hidden}-1 sigmoid on hidden states"
                              if scorer == "gate" else
                              f"mlstm P={w.head_dim // 2} hedgehog, delayed "
                              f"read-out W={w.window}"),
                   "decay": bool(args.decay),
                   "stochastic_eviction": bool(args.stochastic),
                   "flush_mb": args.flush_mb,
                   "parallelism": "none",
                   "timed_window": {
                       "preroll_steps": preroll,
                       "evicting_steps": n_evict,
                       "mean_attention_rows": round(
                           sum(attn_rows(w, n, ev) for n, ev in lens)
                           / steps, 2),
                       "cycle_mean_attention_rows": w.budget + (L - 1) / 2}},
        "step_gbps": round(step_gbps, 1),
        "step_frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "cycles_by_position": (cycle_profile(
            step_ms_all, [ev for _, ev in lens], L, w.batch,
            (w.n0 if args.start_pos is None else args.start_pos)
            + preroll + warmup) if use_events else None),
        "achievable_copy_gbps": None,
        "achievable_read_gbps": None,
        "roofline": roof,
        "timing": timing_note(use_events, flush is not None, args.flush_mb,
                              L, wall, wall_tokens_s),
        "prompt_compress": compress_summary(w, stack, scorer),
        "cpu_baseline": None,
    }
    del stack
    torch.cuda.empty_cache()
    result["achievable_copy_gbps"] = round(achievable_copy_gbps(dev), 1)
    result["achievable_read_gbps"] = round(achievable_read_gbps(dev), 1)
    if not args.no_cpu_baseline:
        cs = args.cpu_steps if args.cpu_steps is not None else max(2 * L, 64)
        cbatch = args.cpu_batch
        if cbatch is None:
            cbatch = 2 if args.scorer == "mlstm" else 16
        cbatch = min(cbatch, w.batch)
        log(f"cpu baseline: oracle on {cbatch} sequences x {cs} steps")
        cb = cpu_baseline(w, args.seed, cbatch, cs, scorer)
        cb["value"] = round(cb["value"], 3)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
