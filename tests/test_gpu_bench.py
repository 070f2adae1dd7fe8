"""bench.py itself on the GPU: its quick modes run in a child process and
print the JSON the measurement contract asks for (a stage's rate with its
roofline fraction; the attainable-rate probes)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_one_stage_line():
    d = _bench("--only", "e2b_global", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "stage_ms", "frac_of_peak"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["dtype"] == "bf16"
    assert set(d["stage_ms"]) == {"e2b_global_prologue", "e2b_global_attn"}
    assert 0.0 < d["e2b_global_prefill_tflops"] < 2500.0
    assert 0.0 < d["frac_of_peak"]["e2b_global_prefill_tflops"] < 1.0


def test_bench_attainable_probes():
    d = _bench("--attainable")
    assert set(d) == {"mfma_loop_bf16_tflops", "mfma_loop_bf16_low_activity_tflops", "stream_read_GBps",
                      "hbm_copy_GBps", "bf16_gemm_8192_tflops"}
    # measured ceilings below the published peaks (2.5 PF/s bf16 dense, 8 TB/s), and not absurdly low
    assert 500.0 < d["mfma_loop_bf16_tflops"] <= d["mfma_loop_bf16_low_activity_tflops"] * 1.02
    assert d["mfma_loop_bf16_low_activity_tflops"] < 2600.0
    assert 2000.0 < d["stream_read_GBps"] < 8200.0

