"""bench.py's command-line contract on a machine without a GPU: one GPU
only (any other --gpus exits with a message), and a JSON error line, not a
number, when no device is visible."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    return p.returncode, lines


def test_more_than_one_gpu_is_refused():
    rc, lines = _run("--gpus", "2")
    assert rc == 2
    msg = json.loads(lines[-1])
    assert "one GPU" in msg["error"]


def test_no_visible_gpu_reports_an_error():
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is visible")
    rc, lines = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert rc == 1
    assert "error" in json.loads(lines[-1])


def test_flush_needs_per_step_events():
    rc, lines = _run("--flush-mb", "512", "--no-kernel-events")
    assert rc == 2
    assert "--flush-mb" in json.loads(lines[-1])["error"]


def test_explicit_preroll_keeps_an_eviction_in_timed_windows():
    # 20 timed steps after 3 + 5 untimed ones end at step 28 < L = 128
    for args in (["--preroll", "3", "--steps", "20", "--warmup", "5"],
                 ["--no-kernel-events", "--preroll", "-1"]):
        rc, lines = _run(*args)
        assert rc == 2
        assert "--preroll" in json.loads(lines[-1])["error"]


def test_window_has_eviction():
    import bench
    assert bench.window_has_eviction(128, 0, 0, 128)      # t = 1..128
    assert not bench.window_has_eviction(128, 0, 0, 127)
    assert not bench.window_has_eviction(128, 128, 0, 127)  # t = 129..255
    assert bench.window_has_eviction(128, 127, 0, 1)      # t = 128
    assert bench.window_has_eviction(1, 0, 0, 1)
    for L, pre, wu, st in [(128, 55, 8, 128), (256, 119, 8, 256), (64, 27, 4, 64)]:
        assert bench.window_has_eviction(L, pre, wu, st)
    for L in (1, 64, 128, 256):
        for wu in (0, 5, 128):
            for st in (1, 20, 512):
                pre = bench.preroll_steps(L, wu, st)
                assert bench.window_has_eviction(L, pre, wu, st)


def test_cycle_profile_sums_whole_cycles():
    import bench
    L = 4
    ev = [False, True, False, False, False, True, False, False, False, True]
    ms = [1.0] * 10
    ms[5] = 3.0
    prof = bench.cycle_profile(ms, ev, L, batch=8, pos0=100)
    # cycles end at steps 5 and 9 (step 1 has no L steps before it)
    assert [p["start_pos"] for p in prof] == [102, 106]
    assert prof[0]["tokens_per_s"] == round(8 * 4 / 6e-3, 1)
    assert prof[1]["tokens_per_s"] == round(8 * 4 / 4e-3, 1)
    many = bench.cycle_profile([1.0] * 400, [(i + 1) % 4 == 0 for i in range(400)],
                               4, 1, 0, max_points=8)
    assert len(many) == 8 and many[0]["start_pos"] == 0
    assert many[-1]["start_pos"] == 396


def test_algorithmic_byte_accounting():
    """The bytes the roofline divides by, written out by hand for the
    batch-96 Qwen3-4B layer (768 slices, d 128, bf16, G 4): per slice, n K
    and V rows of 256 bytes each, 4 bf16 q rows in, 4 float32 output rows
    out, and with the fused append one new K/V row stored plus its
    position."""
    sys.path.insert(0, ROOT)
    import bench
    import synthetic as syn
    w = syn.workload(4)
    per_slice = 1088 * 2 * 256 + 4 * 256 + 4 * 512 + (2 * 256 + 4)
    assert bench.attn_launch_bytes(w, 1088, True) == 768 * per_slice
    assert bench.attn_launch_bytes(w, 1024, False) == \
        768 * (1024 * 2 * 256 + 4 * 256 + 4 * 512)
    # an eviction step besides its attention: append, scoring of L rows,
    # select over the candidates, compaction of the moved rows
    moved = 1000
    extra = bench.evict_extra_bytes(w, 1152, moved)
    append = 768 * (2 * 256 * 2 + 4)
    score = 768 * 128 * (2 * 256 + 4) + 8 * (256 * 64 * 2 + 64 * 4)
    select = 768 * ((1152 - 4 - 128) * 8 + 1024 * 4)
    compact = moved * 2 * (2 * 256 + 8)
    assert extra == append + score + select + compact


def _window(L, warmup, steps):
    """Which timed steps evict, stepping a cache from B entries through the
    pre-roll and the warm-up the way bench.py does (the t-th step after the
    prompt compression evicts when t is a multiple of L)."""
    sys.path.insert(0, ROOT)
    import bench
    p = bench.preroll_steps(L, warmup, steps)
    assert 0 <= p < L
    return [(p + warmup + 1 + s) % L == 0 for s in range(steps)]


def test_timed_window_holds_an_eviction_at_any_step_count():
    # the driver's short run, the default four cycles, the Qwen2.5-14B
    # gate's L = 64, batch 8's L = 256 and the per-token eviction (L = 1)
    for L, warmup, steps in [(128, 5, 20), (128, 128, 512), (64, 5, 20),
                             (256, 0, 1), (256, 3, 7), (1, 5, 20),
                             (128, 300, 2)]:
        ev = _window(L, warmup, steps)
        # the middle step evicts, and so does every L-th step from it
        assert ev == [(s - steps // 2) % L == 0 for s in range(steps)], \
            (L, warmup, steps)
    # whole cycles: exactly one eviction per L steps
    assert sum(_window(128, 128, 512)) == 4


def test_cycle_fold_weighs_one_evicting_step_in_L():
    sys.path.insert(0, ROOT)
    import bench
    L = 128
    ev = _window(L, 5, 20)
    times = [3.0 if e else 1.0 for e in ev]
    # one evicting step of 3 ms and L - 1 steps of 1 ms per cycle
    assert abs(bench.cycle_fold(times, ev, L) - (3.0 + 127.0)) < 1e-12
    # over whole cycles the fold equals the window's time per cycle
    ev = _window(L, 128, 512)
    times = [5.0 if e else 2.0 + 0.001 * i for i, e in enumerate(ev)]
    assert abs(bench.cycle_fold(times, ev, L) - sum(times) / 4) < 0.5
    # L = 1: every step evicts
    assert bench.cycle_fold([2.0, 4.0], [True, True], 1) == 3.0
    import pytest
    with pytest.raises(ValueError):
        bench.cycle_fold([1.0, 1.0], [False, False], L)


def test_cycle_bytes_sum_the_steps_of_one_cycle():
    """One cycle of the batch-96 stack: L - 1 fused-append attentions at
    B + 1 .. B + L - 1 rows, then the evicting step's extras and its
    attention over B rows, in each of the 36 layers."""
    sys.path.insert(0, ROOT)
    import bench
    import synthetic as syn
    w = syn.workload(4)
    B, L = 1024, 128
    moved = {(0, 0): 1000, (1, 0): 1002}
    per_slice_rows = sum(range(B + 1, B + L)) * 2 * 256
    per_slice_fixed = (L - 1) * (4 * 256 + 4 * 512 + 2 * 256 + 4)
    attn = 768 * (per_slice_rows + per_slice_fixed)
    evict = bench.evict_extra_bytes(w, B + L, 1001) + \
        768 * (B * 2 * 256 + 4 * 256 + 4 * 512)
    assert bench.cycle_bytes(w, [], moved, "mlp") == 36 * (attn + evict)
