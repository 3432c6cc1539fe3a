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
