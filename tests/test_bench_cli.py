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
