"""Every buffer a decode run writes stays within its bounds: each of them
(K, V, score, pos, the kept slots, the workspace, the outputs, the pending
hidden states) is a view into a larger allocation whose 64 KiB margins on
both sides hold a sentinel byte pattern. Full eviction cycles of kve_step,
and the one-shot prompt compression, run on the workload shapes (one layer
each); afterwards every margin must still hold the pattern. An off-by-a-row
write by any kernel of the path (append, scorer, select, compaction,
attention, split merge) would land in a margin."""
import numpy as np
import pytest

from kvharness import kve

pytestmark = pytest.mark.gpu

GUARD = 64 << 10
SENTINEL = 0x5A


class Guarded:
    """Device tensors carved out of guarded allocations."""

    def __init__(self, dev):
        self.dev = dev
        self.blocks = []

    def alloc(self, shape, dtype):
        import torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.uint8,
                         device=self.dev)
        self.blocks.append((raw, n))
        return raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, what):
        import torch
        for i, (raw, n) in enumerate(self.blocks):
            lo, hi = raw[:GUARD], raw[GUARD + n:]
            assert bool((lo == SENTINEL).all()), f"{what}: margin below buffer {i}"
            assert bool((hi == SENTINEL).all()), f"{what}: margin above buffer {i}"
        torch.cuda.synchronize()


def _layer(k, g, shape, fill_len, rng_seed):
    """A guarded cache whose first fill_len slots hold random rows,
    positions 0..fill_len-1 and random scores (all scored)."""
    import torch
    gen = torch.Generator(device=g.dev).manual_seed(rng_seed)
    b, H, cap, d = shape.batch, shape.n_kv_heads, shape.capacity, shape.head_dim
    dt = shape.torch_dtype
    c = k.CacheTensors(g.alloc((b, H, cap, d), dt), g.alloc((b, H, cap, d), dt),
                       g.alloc((b, H, cap), torch.float32),
                       g.alloc((b, H, cap), torch.int32))
    c.k.copy_(torch.randn((b, H, cap, d), generator=gen, device=g.dev).to(dt))
    c.v.copy_(torch.randn((b, H, cap, d), generator=gen, device=g.dev).to(dt))
    c.score.copy_(torch.randn((b, H, cap), generator=gen, device=g.dev))
    c.pos.copy_(torch.arange(cap, dtype=torch.int32, device=g.dev)
                .expand(b, H, cap))
    c.pos[:, :, fill_len:] = -1
    return c


CASES = [
    # batch, H, G, B, L, S, W, scorer, steps: the batch-8 B = 2048 layer (the
    # scorer, then select fused with compaction), a batch-96 layer (scoring,
    # select and compaction in one launch), the Qwen2.5-14B layer (hidden-state
    # gate, the LDS-key select, the global compaction, 32-way split merge)
    (8, 8, 4, 2048, 256, 4, 256, "mlp", 560),
    (96, 8, 4, 1024, 128, 4, 128, "mlp", 300),
    (1, 8, 5, 39321, 64, 4, 512, "gate", 140),
]


@pytest.mark.parametrize("case", CASES, ids=["b8-B2048", "b96-B1024",
                                             "qwen2.5-14b-gate"])
def test_decode_writes_stay_in_bounds(case):
    import torch
    k = kve()
    dev = torch.device("cuda")
    batch, H, G, B, L, S, W, scorer, steps = case
    print(f"[bounds] {case}", flush=True)
    g = Guarded(dev)
    d = 128
    shape = k.Shape(batch, H, G, d, B + L, k.BF16)
    pol = k.Policy(B, S, W, L)
    c = _layer(k, g, shape, B, 7)
    gen = torch.Generator(device=dev).manual_seed(11)
    hid = None
    if scorer == "mlp":
        w1 = (torch.randn((H, 64, 2 * d), generator=gen, device=dev) *
              (2 * d) ** -0.5).to(torch.bfloat16)
        sc = k.Scorer.mlp(w1, torch.randn((H, 64), generator=gen, device=dev))
    else:
        D = 5120
        sc = k.Scorer.gate((torch.randn((H, D), generator=gen, device=dev) *
                            D ** -0.5).to(torch.bfloat16))
        hid = g.alloc((batch, L, D), torch.bfloat16)
        hid.zero_()
    ws = g.alloc((k.kve_workspace_bytes(shape, shape.capacity) // 4,),
                 torch.int32)
    out = g.alloc((batch, H * G, d), torch.float32)
    lse = g.alloc((batch, H * G), torch.float32)
    keep = g.alloc((batch, H, B), torch.int32)
    st = k.DecodeState(B, B, B)
    evictions = 0
    for i in range(steps):
        kn = torch.randn((batch, H, d), generator=gen, device=dev).to(torch.bfloat16)
        vn = torch.randn((batch, H, d), generator=gen, device=dev).to(torch.bfloat16)
        q = torch.randn((batch, H * G, d), generator=gen, device=dev).to(torch.bfloat16)
        if scorer == "mlp":
            k.kve_step(shape, pol, sc, c, st, kn, vn, q, out, lse, keep, ws)
        else:
            hn = torch.randn((batch, 5120), generator=gen, device=dev).to(
                torch.bfloat16)
            k.kve_step(shape, pol, sc, c, st, kn, vn, q, out, lse, keep, ws,
                       hidden_new=hn, hidden_buf=hid)
        evictions += st.evicted
    torch.cuda.synchronize()
    assert evictions >= 2
    assert bool(torch.isfinite(out).all())
    g.check(f"{case}")


def test_prompt_compression_writes_stay_in_bounds():
    """The batch-8 prompt compression: 8192 entries per slice to 2048 (the
    select that keeps the keys in LDS, then the LDS-bitmap compaction)."""
    import torch
    k = kve()
    dev = torch.device("cuda")
    g = Guarded(dev)
    shape = k.Shape(8, 8, 4, 128, 8192, k.BF16)
    c = _layer(k, g, shape, 8192, 3)
    keep = g.alloc((8, 8, 2048), torch.int32)
    pol = k.Policy(2048, 4, 256, 256)
    k.kve_select_evict(shape, pol, c, 8192, 2048, keep)
    k.kve_compact(shape, c, 8192, keep, 2048)
    torch.cuda.synchronize()
    g.check("prompt compression")
