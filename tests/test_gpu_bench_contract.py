"""bench.py's JSON line on a GPU: one line with every field its readers expect (the metric,
the step timing, the workload, the dominant kernel's roofline with its measured traffic
and the oracle's CPU baseline), from a short run of the default MoE step."""

import json
import os
import subprocess
import sys

import pytest

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_default_line():
    require_gpu()
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "3"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    say(f"[bench] {d['value']} {d['unit']}, {d['ms_per_step']} ms per step")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 3
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert "workload" in d["config"] and "model" not in d["config"]
    # value: the step's GEMM flops over its time
    assert abs(d["value"] - d["step_gemm_gflop"] / d["ms_per_step"]) <= 0.01 * d["value"]
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 5000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the dominant kernel's achieved rate is its flops over its measured launch time
    assert abs(roof["achieved"] - roof["flops_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e12) <= 0.01 * roof["achieved"]
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1

