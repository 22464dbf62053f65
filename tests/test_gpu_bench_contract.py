"""The line bench.py prints, from a short run on the GPU: one JSON object with the fields
the measurement contract names, the whole step's kept-tile rate as its value, and the
dominant kernel's roofline entry."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def test_bench_line_fields():
    print("bench.py --steps 2 --warmup 1 --no-cpu", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--no-cpu"],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 2 and rec["warmup"] == 1
    assert rec["unit"] == "TFLOP/s" and rec["higher_is_better"] is True and rec["vs_baseline"] is None
    assert rec["dtype"] == "bf16" and rec["data"].startswith("synthetic")
    # the headline workload is the largest single-GPU one; the 480p layer rides along
    assert rec["config"]["workload"] == "wan14b_720p_cfg"
    extra = rec["extra_workloads"]["wan1.3b_480p"]
    assert extra["config"]["workload"] == "wan1.3b_480p" and extra["value"] > 0 and extra["ms_per_step"] > 0
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    # the value is the whole step's rate: kept-tile FLOPs over the step time, so it
    # cannot exceed the attention kernel's own rate
    assert rec["value"] <= rec["attn_tflops"] * 1.001
    roof = rec["roofline"]
    assert set(roof) == {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1
    # HBM bytes per launch: at least Q + K + V + O once (4 x 80 x 80640 x 128 x 2 bytes)
    assert roof["traffic"] is None or roof["traffic"] >= 4 * 80 * 80640 * 128 * 2
    assert rec["kept_tiles"] * 4 * 64 * 64 * 128 == pytest.approx(roof["achieved"] * 1e12 * rec["ms_attn"] * 1e-3, rel=1e-3)
    assert "cpu_baseline" not in rec       # --no-cpu
