"""bench.py's command-line contract on a machine without a GPU: more than one GPU is
refused with exit status 2 and a message naming the reason, and a run with no GPU fails
loudly rather than falling back to the CPU."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""          # no JSON line


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_no_gpu_fails_loudly():
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode != 0
    assert "GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_only_for_its_workload_and_kernel():
    """The committed counter figure belongs to one kernel on one workload: any other
    bench line reports its traffic as unknown rather than borrowing it."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.read_traffic("wan1.3b_480p", "attn_fwd_bf16_kernel<128, raster>")
    assert t is None or t > 0
    assert bench.read_traffic("tiny", "attn_fwd_f32_kernel<64, raster>") is None
    assert bench.read_traffic("wan1.3b_480p", "attn_fwd_bf16_kernel<128, fractal>") is None
    assert bench.read_traffic("hunyuan_720p_sta", "attn_fwd_bf16_kernel<128, raster>") is None
