"""bench.py's command-line contract on a machine without a GPU: more than one GPU is
refused with exit status 2 and a message naming the reason, and a run with no GPU fails
loudly rather than falling back to the CPU."""
import glob
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
    """Each committed counter figure belongs to one kernel on one workload: any other
    bench line reports its traffic as unknown rather than borrowing it."""
    sys.path.insert(0, ROOT)
    import bench
    files = sorted(glob.glob(os.path.join(bench.PROFILES, "attn_fwd_bf16_*_traffic.txt")))
    assert files, "no committed traffic summary"
    owners = []
    for path in files:
        kv = {}
        for ln in open(path):
            if ":" in ln and not ln.lstrip().startswith("#"):
                key, val = ln.split(":", 1)
                kv[key.strip()] = val.strip()
        assert path == bench.traffic_file(kv["workload"])
        owners.append((kv["workload"], kv["kernel"]))
        t = bench.read_traffic(kv["workload"], kv["kernel"])
        # valid only while the kernel source is the one the counters were taken on
        if kv["kernel_source_sha256"] == bench.kernel_source_hash():
            assert t == float(kv["hbm_bytes_per_launch"]) > 0
        else:
            assert t is None
    for other in [("tiny", "attn_fwd_f32_kernel<64, raster>"), ("wan14b_720p_cfg", "attn_fwd_bf16_kernel<128, fractal>"),
                  ("hunyuan_720p_sta", "attn_fwd_bf16_kernel<128, raster>"), ("wan1.3b_480p", "attn_fwd_bf16_kernel<128, fractal>"),
                  ("wan14b_720p_cfg", "attn_fwd_bf16_kernel<128, raster>"), ("wan1.3b_480p", "attn_fwd_bf16_kernel<128, raster>")]:
        if other not in owners:
            assert bench.read_traffic(*other) is None, other


def test_cpu_baseline_is_bounded_and_extrapolated():
    """The oracle baseline on a tiny budget: a sample of heads and query blocks, scaled
    to the whole step and flagged as extrapolated."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import get_config, make_qkv
    cfg = get_config("wan1.3b_480p")
    q, k, v = make_qkv(cfg, pairs=[(0, 0), (0, cfg.heads - 1)])
    cb = bench.cpu_baseline(cfg, q, k, v, kept_flops_total=1.0e6 * 4 * 64 * 64 * 128, budget_s=0.5,
                            blocks_per_head=4)
    assert cb["extrapolated"] is True and cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "of 12 (batch, head) slices" in cb["sample"]
