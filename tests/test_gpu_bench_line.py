"""bench.py prints one JSON line with every field of its contract in each of
its modes (decode with the per-step cycle fold and the attention roofline,
the oracle's CPU baseline, prefill at both prefill shapes, the sink gate),
run here with few steps; --hw-reference prints its reference measurements."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric": str, "value": (int, float), "unit": str, "n_gpus": int,
        "steps": int, "warmup": int, "ms_per_step": (int, float),
        "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
        "config": dict}
ROOF = {"bound": str, "achieved": (int, float), "peak": (int, float),
        "unit": str, "frac": (int, float)}
CPU = {"value": (int, float), "unit": str, "cores": int, "kind": str,
       "sample": str}

MODES = [
    ("decode-1layer", ["--workload", "qwen3-4b-1layer-b16", "--steps", "8",
                       "--warmup", "2", "--no-cpu-baseline"], True, False),
    ("decode-tiny-cpu", ["--workload", "tiny-1layer-fp32", "--steps", "4",
                         "--warmup", "1", "--cpu-batch", "1", "--cpu-steps",
                         "8"], False, True),
    ("prefill", ["--prefill", "--steps", "1", "--warmup", "0",
                 "--no-cpu-baseline"], True, False),
    ("sink-gate", ["--sink-gate", "--steps", "2", "--warmup", "1",
                   "--no-cpu-baseline"], True, False),
    ("prefill-14b", ["--prefill", "--workload", "qwen2.5-14b-48layer-131k-gate",
                     "--steps", "1", "--warmup", "0", "--no-cpu-baseline"],
     True, False),
]


@pytest.mark.parametrize("mode", MODES, ids=[m[0] for m in MODES])
def test_bench_line_contract(mode):
    name, args, roofline, cpu = mode
    print(f"[bench-line] {name}", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    for key, typ in KEYS.items():
        assert isinstance(d.get(key), typ), key
    assert d["n_gpus"] == 1 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["vs_baseline"] is None
    assert "workload" in d["config"]
    if roofline:
        r = d["roofline"]
        for key, typ in ROOF.items():
            assert isinstance(r.get(key), typ), key
        assert "traffic" in r
        assert 0 < r["frac"] <= 1.0
        assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if cpu:
        c = d["cpu_baseline"]
        for key, typ in CPU.items():
            assert isinstance(c.get(key), typ), key
        assert c["kind"] == "oracle" and c["value"] > 0
    else:
        assert d["cpu_baseline"] is None


def test_hw_reference_line():
    """--hw-reference prints one JSON object: the issue probe's times per
    mode and the vendor libraries' GEMM and attention rates."""
    print("[bench-line] hw-reference", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--hw-reference"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    probe = d["issue_probe"]["ns_per_simd_iteration"]
    for mode in ("mfma", "fma", "mfma_and_fma_two_waves",
                 "mfma_and_fma_one_wave", "exp", "mfma_and_exp_two_waves",
                 "mfma_and_exp_one_wave"):
        assert probe[mode] > 0, mode
    # two kinds of work on one SIMD never take less than the longer part
    assert probe["mfma_and_fma_two_waves"] >= 0.95 * max(probe["mfma"],
                                                          probe["fma"])
    for name, r in d["library_reference"].items():
        assert r["ms"] > 0 and 0 < r["frac"] <= 1.0, name
