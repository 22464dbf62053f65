"""Benchmark of the NABLA forward path on one MI355X.

One step = the whole path on one layer's worth of synthetic video-shaped Q/K/V
already resident in HBM, raster order in and out: fractal flattening -> block mask
(pooling, pooled map, softmax, CDF cutoff, lists) -> block-sparse attention -> inverse
flattening of O.  The timed step runs the raster-order entry points, which apply the
flattening in the kernels' addressing; the same step with explicit reorder passes
(nabla_reorder before and after) is timed in the same run and reported beside it.

The default workload is the largest one that fits one GPU: the Wan2.1-14B-like 720p
layer with its classifier-free-guidance batch (B 2, 40 heads, 21 x 48 x 80 latent grid);
the Wan2.1-1.3B-like 480p layer is measured in the same run and reported under
``extra_workloads``.

Prints one JSON line.  ``value`` is kept-tile TFLOP/s over the whole step
(4 N^2 d FLOP per kept 64 x 64 tile / step time); the sub-phase times, the
attention kernel's own TFLOP/s against the bf16 MFMA peak and the mask phase's
GB/s against HBM peak ride along, with the oracle timed on the host beside it.

    python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu] [--no-extra]
    python bench.py --no-cpu --loop-seconds 12      # steady load for power / clock readings
    python bench.py --gemm-reference                # dense bf16 GEMM of the vendor library
    python bench.py --config 1 --backward --no-cpu  # the gradient of the attention step
    python bench.py --config 1 --sip 185 --no-cpu   # SIP selection + weighted attention
    python bench.py --config 1 --ibcs --no-cpu      # IBCS block scores + attention
    python bench.py --config 1 --ibcs --sip 185 --no-cpu   # SIP sampling from IBCS scores
    python bench.py --config 1 --mask-every 4 --no-cpu     # mask rebuilt every 4th step
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_sparse_attention_blockmean_amd as nab  # noqa: E402
from synth import GENERATOR_VERSION, get_config, make_qkv  # noqa: E402

METRIC = "block-sparse attn ms/layer + kept-tile TFLOP/s (% MFMA peak); mask GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_blockmean_amd", "csrc", "attn_bf16.hip")
ATTN_TILE = os.path.join(ROOT, "block_sparse_attention_blockmean_amd", "csrc", "attn_tile.h")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(workload: str) -> str:
    """The committed --pmc summary of the attention kernel on one workload."""
    return os.path.join(PROFILES, f"attn_fwd_bf16_{workload}_traffic.txt")


def kernel_source_hash() -> str:
    """Hash of the attention kernel's sources (the kernel file and the tile header)."""
    h = hashlib.sha256()
    for path in (ATTN_SRC, ATTN_TILE):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """HBM bytes per attention launch from the committed --pmc summary, valid only
    if it was taken on the current kernel source, for this workload and this kernel."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.lstrip().startswith("#"):
            key, val = ln.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if kv.get("workload") != workload or kv.get("kernel") != kernel:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, q, k, v, kept_flops_total, budget_s=20.0, blocks_per_head=48):
    """The oracle (untuned) on a bounded sample of the same workload, extrapolated to one
    whole step.  Heads are taken in a seeded order (first, last, then the rest shuffled);
    for each, the oracle's reorder of Q, K, V and its float32 mask, then float64 attention
    of a seeded sample of the head's query blocks over their kept tiles, until the budget
    is spent.  Mask time is scaled by the head count, attention time by the kept-tile
    count of the whole step."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    G, nb = cfg.BH, cfg.nb
    scale = 1.0 / np.sqrt(cfg.d)
    rng = np.random.default_rng(1000 + cfg.index)
    order = [0] + ([G - 1] if G > 1 else []) + [int(x) for x in rng.permutation(np.arange(1, G - 1))]
    t_mask = t_attn = 0.0
    heads = blocks = tiles = 0
    t_start = time.perf_counter()
    for g in order:
        b, h = divmod(g, cfg.heads)
        t0 = time.perf_counter()
        qn, kn, vn = (t[b, h].float().numpy() for t in (q, k, v))
        qf, kf, vf = (O.reorder(a, cfg.T, cfg.H, cfg.W, cfg.P) for a in (qn, kn, vn))
        mk = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, cfg.sta)
        t_mask += time.perf_counter() - t0
        heads += 1
        for i in rng.choice(nb, size=min(nb, blocks_per_head), replace=False):
            t0 = time.perf_counter()
            O.attention_block(qf, kf, vf, mk["mask"][i], int(i), cfg.N, scale)
            t_attn += time.perf_counter() - t0
            blocks += 1
            tiles += int(mk["mask"][i].sum())
            if time.perf_counter() - t_start > budget_s:
                break
        if time.perf_counter() - t_start > budget_s:
            break
    kept_total = kept_flops_total / (4.0 * cfg.N * cfg.N * cfg.d)
    t_step = t_mask * G / heads + t_attn * kept_total / max(tiles, 1)
    whole = heads == G and blocks == G * nb
    return {
        "value": kept_flops_total / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "extrapolated": not whole,
        "sample": (f"oracle reorder + float32 mask on {heads} of {G} (batch, head) slices ({t_mask:.1f} s), "
                   f"float64 attention of {blocks} seeded query blocks over their {tiles} kept tiles "
                   f"({t_attn:.1f} s); scaled by head count and by kept tiles ({kept_total:.0f} in the step) "
                   f"to est. {t_step:.0f} s per step"),
        "est_s_per_step": t_step,
    }


def bench_backward(args, cfg, qd, kd, vd) -> int:
    """Gradient of the attention step on the same workload, in the step's token order
    (raster in and out, the flattening applied in the addressing, when N == P*P): the
    mask and the forward (with its log-sum-exp) run once untimed; then K calls of
    block_sparse_attn_bwd(_raster) (row dots, transposed lists, start orders, the dQ
    sweep and the dK/dV sweep), each bracketed by HIP events on the launch stream."""
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    raster = N == P * P
    g = torch.Generator(device="cuda").manual_seed(1234)
    dout = torch.randn(qd.shape, device="cuda", generator=g).to(qd.dtype)
    if raster:
        qf, kf, vf, dof = qd, kd, vd, dout
        cnt, idx, sched = nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True, raster=True)
        o, lse = nab.attn_fwd_raster(qf, kf, vf, cnt, idx, T, H, W, P, N, schedule=sched, with_lse=True)
    else:
        qf, kf, vf, dof = (nab.reorder(t, T, H, W, P) for t in (qd, kd, vd, dout))
        cnt, idx, sched = nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True)
        o, lse = nab.attn_fwd(qf, kf, vf, cnt, idx, N, schedule=sched, with_lse=True)
    ws = torch.empty(nab.attn_bwd_workspace_size(cfg.B, cfg.heads, cfg.L, N), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = (torch.empty_like(qf) for _ in range(3))

    def call():
        nab.attn_bwd(qf, kf, vf, o, dof, lse, cnt, idx, N, workspace=ws, dq=dq, dk=dk, dv=dv,
                     raster=(T, H, W, P) if raster else None)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    kept = int(cnt.sum().item())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    alg = kept * 10.0 * N * N * cfg.d          # five products of 2 N^2 d per kept tile
    exe = kept * 14.0 * N * N * cfg.d          # seven: S and dP are formed in both sweeps
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    rec = {
        "metric": "block-sparse attn backward (dQ, dK, dV) kept-tile TFLOP/s",
        "value": round(alg / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({GENERATOR_VERSION}), dO ~ N(0, 1) seeded",
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.heads, "d": cfg.d, "L": cfg.L,
                   "blocks_per_head": cfg.nb, "thr": cfg.thr},
        "ms_bwd": round(ms, 4),
        "kept_fraction": round(kept / (cfg.BH * cfg.nb * cfg.nb), 5),
        "flop_convention": "algorithmic 10 N^2 d per kept tile (5 products); executed 14 N^2 d",
        "order": "raster, flattening in the addressing" if raster else "fractal (explicit reorder before)",
        "executed_tflops": round(exe / (ms * 1e-3) / 1e12, 2),
        "executed_frac_of_peak": round(exe / (ms * 1e-3) / 1e12 / peak, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_sip(args, cfg, qd, kd, vd) -> int:
    """SIP variant of the step on fractal-order tensors: nabla_build_mask_sip (pooling,
    pooled map, inclusion probabilities, sampling against seeded draws) - or with --ibcs
    nabla_build_mask_ibcs_sip (IBCS scores of 128-query clusters, then the same
    sampling) - and block_sparse_attn_fwd_weighted, each bracketed by HIP events."""
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    qf, kf, vf = (nab.reorder(t, T, H, W, P) for t in (qd, kd, vd))
    g = torch.Generator(device="cuda").manual_seed(4321)
    u = torch.rand((cfg.B, cfg.heads, cfg.nb, cfg.nb), device="cuda", generator=g)
    ws = torch.empty(nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, N, ibcs=args.ibcs),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(qf)
    state = {}

    def mask():
        state["lists"] = nab.build_mask_sip(qf, kf, T, H, W, P, args.sip, u, N, with_schedule=True, workspace=ws,
                                            ibcs=args.ibcs)

    def attn():
        cnt, idx, logw, sched = state["lists"]
        nab.attn_fwd_weighted(qf, kf, vf, cnt, idx, logw, N, out=o, schedule=sched)

    for _ in range(args.warmup):
        mask()
        attn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        mask()
        e[1].record()
        attn()
        e[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_mask = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    kept = int(state["lists"][0].sum().item())
    flops = kept * 4.0 * N * N * cfg.d
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    rec = {
        "metric": ("IBCS+SIP" if args.ibcs else "SIP") + " block-sparse attn: kept-tile TFLOP/s (weighted attention), ms/layer",
        "value": round(flops / (ms_attn * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({GENERATOR_VERSION}), draws U[0,1) seeded",
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.heads, "d": cfg.d, "L": cfg.L,
                   "blocks_per_head": cfg.nb, "budget": args.sip, "scores": "ibcs_q128" if args.ibcs else "pooled"},
        "ms_mask_sip": round(ms_mask, 4),
        "ms_attn_weighted": round(ms_attn, 4),
        "mean_kept_per_row": round(kept / (cfg.BH * cfg.nb), 2),
        "attn_frac_of_peak": round(flops / (ms_attn * 1e-3) / 1e12 / peak, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_ibcs(args, cfg, qd, kd, vd) -> int:
    """IBCS variant of the step on raster-order tensors, the fractal flattening applied
    in the addressing as in the default step: nabla_build_mask_ibcs_raster (K pooling,
    8 clusters per group of 128 queries as on the AB-Attention page, centroid map, CDF
    cut, lists) and block_sparse_attn_fwd_raster on its lists, each bracketed by HIP
    events; the IBCS mask with 64-query groups and the plain NABLA mask on the same
    inputs are timed beside it."""
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    qf, kf, vf = qd, kd, vd      # raster order
    ws = torch.empty(nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, N, ibcs=True, ibcs_group=64),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(qf)
    state = {}

    def mask():
        state["lists"] = nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True,
                                        workspace=ws, ibcs=True, ibcs_group=128, raster=True)

    def mask_nabla():
        nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True, workspace=ws, raster=True)
        nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True, workspace=ws, ibcs=True,
                       ibcs_group=64, raster=True)

    def attn():
        cnt, idx, sched = state["lists"]
        nab.attn_fwd_raster(qf, kf, vf, cnt, idx, T, H, W, P, N, out=o, schedule=sched)

    for _ in range(args.warmup):
        mask()
        attn()
        mask_nabla()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        mask()
        e[1].record()
        attn()
        e[2].record()
        nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True, workspace=ws, raster=True)
        e[3].record()
        nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True, workspace=ws, ibcs=True,
                       ibcs_group=64, raster=True)
        e[4].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_mask = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_nabla = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    ms_q64 = float(np.mean([e[3].elapsed_time(e[4]) for e in ev]))
    kept = int(state["lists"][0].sum().item())
    flops = kept * 4.0 * N * N * cfg.d
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    rec = {
        "metric": "IBCS block-sparse attn: kept-tile TFLOP/s over mask + attention, ms/layer",
        "value": round(flops / ((ms_mask + ms_attn) * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({GENERATOR_VERSION})",
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.heads, "d": cfg.d, "L": cfg.L,
                   "blocks_per_head": cfg.nb, "thr": cfg.thr, "sta": cfg.sta, "ibcs_query_group": 128,
                   "order": "raster, flattening in the addressing"},
        "ms_mask_ibcs": round(ms_mask, 4),
        "ms_mask_ibcs_query_group_64": round(ms_q64, 4),
        "ms_mask_nabla_same_inputs": round(ms_nabla, 4),
        "ms_attn": round(ms_attn, 4),
        "kept_fraction": round(kept / (cfg.BH * cfg.nb * cfg.nb), 4),
        "attn_frac_of_peak": round(flops / (ms_attn * 1e-3) / 1e12 / peak, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_mask_reuse(args, cfg, qd, kd, vd) -> int:
    """A run of denoising steps in which the mask is rebuilt only every `mask_every`-th
    step and its lists are reused by the steps in between (the AB-Attention page
    recomputes its plan every 4 steps): raster-order entry points, the step's attention
    every step.  Reports the amortised step time; inputs stay the same from step to
    step, which changes no kernel's work."""
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    K = args.mask_every
    nb = cfg.nb
    cnt = torch.empty((cfg.B, cfg.heads, nb), dtype=torch.int32, device="cuda")
    idx = torch.empty((cfg.B, cfg.heads, nb, nb), dtype=torch.int32, device="cuda")
    sched = torch.empty((cfg.BH * nb,), dtype=torch.int32, device="cuda")
    ws = torch.empty(nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, N), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(qd)

    def step(i):
        if i % K == 0:
            nab.build_mask(qd, kd, T, H, W, P, N, cfg.thr, cfg.sta, workspace=ws, kv_count=cnt, kv_index=idx,
                           schedule=sched, raster=True)
        nab.attn_fwd_raster(qd, kd, vd, cnt, idx, T, H, W, P, N, out=o, schedule=sched)

    steps = max(K, (args.steps // K) * K)          # whole mask periods
    for i in range(max(args.warmup, 1) * K):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / steps
    kept = int(cnt.sum().item())
    flops = kept * 4.0 * N * N * cfg.d
    rec = {
        "metric": "NABLA step with the mask reused: kept-tile TFLOP/s over the amortised step",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1) * K,
        "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round((t1 - t0) * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({GENERATOR_VERSION})",
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.heads, "d": cfg.d, "L": cfg.L,
                   "blocks_per_head": nb, "thr": cfg.thr, "sta": cfg.sta, "mask_every": K},
        "kept_fraction": round(kept / (cfg.BH * nb * nb), 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="4", help="workload index or name (default: the Wan-14B-like "
                    "720p layer with its CFG batch, the largest single-GPU workload)")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the Wan-1.3B-like 480p workload that the default run reports as an extra key")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only an identity reorder (P=1, a plain copy) of 1 GiB, for counter scaling")
    ap.add_argument("--loop-seconds", type=float, default=0.0,
                    help="after the warm-up, repeat the step for this long (a progress line per "
                         "second, no JSON line): a steady load for power and clock readings")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradient of the attention step (block_sparse_attn_bwd) instead of "
                         "the forward path; prints its own JSON line")
    ap.add_argument("--sip", type=int, default=0, metavar="BUDGET",
                    help="time the SIP variant instead: sampled selection with this expected number "
                         "of blocks per row and attention with the Horvitz-Thompson logit shifts; "
                         "prints its own JSON line")
    ap.add_argument("--ibcs", action="store_true",
                    help="time the IBCS variant instead: block scores from 8 query clusters per block, "
                         "NABLA's CDF cut, attention on the kept tiles; prints its own JSON line")
    ap.add_argument("--mask-every", type=int, default=0, metavar="K",
                    help="time a run of steps that rebuilds the mask only every K-th step and reuses "
                         "its lists in between; prints its own JSON line")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="time only a dense 8192^3 bf16 GEMM of the vendor library (torch.matmul) "
                         "for --loop-seconds (default 10): the rate a plain GEMM sustains on this "
                         "GPU, as context for the attention kernel's MFMA fraction")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path would "
              f"shard by (batch, head), with no exchange between GPUs)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    nab.load_library()

    if args.copy_calibration:
        n = 1 << 29   # 1 GiB of bf16
        x = torch.randn(n // 128, 128, device="cuda").to(torch.bfloat16).reshape(1, 1, -1, 128)
        y = torch.empty_like(x)
        L = x.shape[2]
        for _ in range(max(1, args.steps)):
            nab.reorder(x, 1, 1, L, 1, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": x.numel() * 2,
                          "copy_calibration_bytes_written": y.numel() * 2, "launches": args.steps}))
        return 0

    if args.gemm_reference:
        n = 8192
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        secs = args.loop_seconds if args.loop_seconds > 0 else 10.0
        t0 = time.perf_counter()
        rates = []
        while time.perf_counter() - t0 < secs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                torch.matmul(a, b, out=c)
            e1.record()
            torch.cuda.synchronize()
            rates.append(2.0 * n ** 3 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12)
            print(f"# t={time.perf_counter() - t0:.1f}s gemm {rates[-1]:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)
        tail = rates[len(rates) // 2:]
        print(json.dumps({"gemm_reference": "torch.matmul bf16 (hipBLASLt)", "m": n, "n": n, "k": n,
                          "tflops_steady": round(float(np.mean(tail)), 1), "seconds": round(secs, 1)}))
        return 0

    cfg = get_config(int(args.config) if args.config.isdigit() else args.config)
    say(f"# workload {cfg.name}: B{cfg.B} heads{cfg.heads} d{cfg.d} {cfg.dtype} "
        f"{cfg.T}x{cfg.H}x{cfg.W} P{cfg.P} N{cfg.N} thr{cfg.thr} sta{cfg.sta}")
    q, k, v = make_qkv(cfg)
    say("# inputs generated")
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))

    if args.backward:
        return bench_backward(args, cfg, qd, kd, vd)
    if args.sip > 0:
        return bench_sip(args, cfg, qd, kd, vd)   # --ibcs picks the IBCS scores
    if args.ibcs:
        return bench_ibcs(args, cfg, qd, kd, vd)
    if args.mask_every > 0:
        return bench_mask_reuse(args, cfg, qd, kd, vd)
    if args.loop_seconds > 0:
        return loop_step(args, cfg, qd, kd, vd)

    m = measure_step(args, cfg, qd, kd, vd)
    kept, kept_flops = m["kept"], m["kept_flops"]
    ms_step, ms_mask, ms_attn = m["ms_step"], m["ms_mask"], m["ms_attn"]
    nb = cfg.nb
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = kept_flops / (ms_attn * 1e-3) / 1e12
    kernel = f"attn_fwd_{'bf16' if cfg.dtype == 'bf16' else 'f32'}_kernel<{cfg.d}, {'raster' if m['raster'] else 'fractal'}>"
    traffic = read_traffic(cfg.name, kernel)

    rec = {
        "metric": METRIC,
        "value": round(kept_flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({GENERATOR_VERSION}: smooth 3D cosine field + N(0,0.5^2) noise, seeded)",
        "config": workload_config(cfg),
        "path": ("raster order in and out, fractal flattening applied in the mask and attention "
                 "kernels' addressing" if m["raster"] else "explicit reorder passes"),
    }
    rec.update(phase_summary(cfg, m))
    rec["roofline"] = {
        # the float32 path computes on plain float32 FMAs (the vector unit)
        "bound": "mfma" if cfg.dtype == "bf16" else "alu",
        "achieved": round(attn_tflops, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / peak, 4),
        "traffic": traffic,
    }
    rec["device"] = torch.cuda.get_device_name(0)
    rec["cus"] = torch.cuda.get_device_properties(0).multi_processor_count

    # the other large workload as an extra key (same step, same counts of steps)
    if args.extra and args.config in ("4", "wan14b_720p_cfg"):
        del qd, kd, vd
        torch.cuda.empty_cache()
        ecfg = get_config("wan1.3b_480p")
        say(f"# extra workload {ecfg.name}")
        eq, ek, ev = (t.to(dev) for t in make_qkv(ecfg))
        em = measure_step(args, ecfg, eq, ek, ev)
        e_attn = em["kept_flops"] / (em["ms_attn"] * 1e-3) / 1e12
        extra = {"config": workload_config(ecfg), "ms_per_step": round(em["ms_step"], 4),
                 "value": round(em["kept_flops"] / (em["ms_step"] * 1e-3) / 1e12, 3)}
        extra.update(phase_summary(ecfg, em))
        extra["attn_frac_of_peak"] = round(e_attn / PEAK_BF16_TFLOPS, 4)
        rec["extra_workloads"] = {ecfg.name: extra}
        del eq, ek, ev
        torch.cuda.empty_cache()

    if not args.no_cpu:
        say("# timing the oracle on the host (bounded sample)")
        cb = cpu_baseline(cfg, q, k, v, kept_flops)
        cb["value"] = float(f"{cb['value']:.3g}")
        rec["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample", "extrapolated")}
    print(json.dumps(rec), flush=True)
    return 0


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def workload_config(cfg) -> dict:
    return {"workload": cfg.name, "B": cfg.B, "heads": cfg.heads, "d": cfg.d, "T": cfg.T, "H": cfg.H,
            "W": cfg.W, "P": cfg.P, "N": cfg.N, "thr": cfg.thr, "sta": list(cfg.sta) if cfg.sta else None,
            "L": cfg.L, "blocks_per_head": cfg.nb}


def phase_summary(cfg, m) -> dict:
    """Per-phase times and rates of one measured step (see measure_step)."""
    esize = 2 if cfg.dtype == "bf16" else 4
    tensor_bytes = cfg.BH * cfg.L * cfg.d * esize
    mask_bytes = 2 * tensor_bytes + 4 * (m["kept"] + cfg.BH * cfg.nb)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = m["kept_flops"] / (m["ms_attn"] * 1e-3) / 1e12
    out = {
        "ms_layer": round(float(m["ms_mask"] + m["ms_attn"]), 4),
        "ms_attn": round(float(m["ms_attn"]), 4),
        "ms_mask": round(float(m["ms_mask"]), 4),
        "gpu_ms_per_step": round(float(m["gpu_ms"]), 4),
        "kept_fraction": round(m["kept"] / (cfg.BH * cfg.nb * cfg.nb), 5),
        "kept_tiles": int(m["kept"]),
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_of_peak": round(attn_tflops / peak, 4),
        "mask_GBps": round(mask_bytes / (m["ms_mask"] * 1e-3) / 1e9, 1),
        "mask_frac_of_hbm": round(mask_bytes / (m["ms_mask"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
    }
    if "ms_step_x" in m:
        out["explicit_reorder_path"] = {
            "ms_per_step": round(m["ms_step_x"], 4),
            "value": round(m["kept_flops"] / (m["ms_step_x"] * 1e-3) / 1e12, 3),
            "ms_reorder_qkv": round(m["ms_reorder_in"], 4),
            "ms_mask": round(m["ms_mask_x"], 4),
            "ms_attn": round(m["ms_attn_x"], 4),
            "ms_reorder_o": round(m["ms_reorder_out"], 4),
        }
        out["reorder_GBps"] = round(3 * 2 * tensor_bytes / (m["ms_reorder_in"] * 1e-3) / 1e9, 1)
    return out


def make_steps(cfg, qd, kd, vd):
    """The timed step (raster-order entry points when N == P*P) and the same path with
    explicit reorder passes, on shared output buffers.  Each takes an optional list of
    events, recorded on torch's current stream, which is the stream every library call
    launches on."""
    dev = qd.device
    qf, kf, vf, of, od = (torch.empty_like(qd) for _ in range(5))
    nb = cfg.nb
    cnt = torch.empty((cfg.B, cfg.heads, nb), dtype=torch.int32, device=dev)
    idx = torch.empty((cfg.B, cfg.heads, nb, nb), dtype=torch.int32, device=dev)
    ws = torch.empty(nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, cfg.N),
                     dtype=torch.uint8, device=dev)
    sched = torch.empty((cfg.BH * nb,), dtype=torch.int32, device=dev)
    T, H, W, P = cfg.T, cfg.H, cfg.W, cfg.P

    def step(ev=None):
        if ev:
            ev[0].record()
        nab.reorder(qd, T, H, W, P, out=qf)
        nab.reorder(kd, T, H, W, P, out=kf)
        nab.reorder(vd, T, H, W, P, out=vf)
        if ev:
            ev[1].record()
        nab.build_mask(qf, kf, T, H, W, P, cfg.N, cfg.thr, cfg.sta, workspace=ws, kv_count=cnt,
                       kv_index=idx, schedule=sched)
        if ev:
            ev[2].record()
        nab.attn_fwd(qf, kf, vf, cnt, idx, cfg.N, out=of, schedule=sched)
        if ev:
            ev[3].record()
        nab.reorder(of, T, H, W, P, inverse=True, out=od)
        if ev:
            ev[4].record()

    # The same path with the fractal flattening folded into the kernels' addressing
    # (raster-order entry points, N == P*P): no reorder pass, bit-identical output.
    def step_raster(ev=None):
        if ev:
            ev[0].record()
        nab.build_mask(qd, kd, T, H, W, P, cfg.N, cfg.thr, cfg.sta, workspace=ws, kv_count=cnt,
                       kv_index=idx, schedule=sched, raster=True)
        if ev:
            ev[1].record()
        nab.attn_fwd_raster(qd, kd, vd, cnt, idx, T, H, W, P, cfg.N, out=od, schedule=sched)
        if ev:
            ev[2].record()

    raster = cfg.N == P * P
    return step, (step_raster if raster else None), cnt


def measure_step(args, cfg, qd, kd, vd) -> dict:
    """Warm-up, then args.steps timed steps of each form of the step (wall clock between
    synchronisations; per-phase times from HIP events on the launch stream)."""
    step, step_raster, cnt = make_steps(cfg, qd, kd, vd)
    raster = step_raster is not None
    for _ in range(args.warmup):
        step()
        if raster:
            step_raster()
    torch.cuda.synchronize()
    kept = int(cnt.sum().item())
    m = {"kept": kept, "kept_flops": kept * 4.0 * cfg.N * cfg.N * cfg.d, "raster": raster}

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    phase = np.mean([[ev[i].elapsed_time(ev[i + 1]) for i in range(4)] for ev in events], axis=0)
    m["ms_reorder_in"], m["ms_mask_x"], m["ms_attn_x"], m["ms_reorder_out"] = (float(x) for x in phase)
    m["ms_step_x"] = (t1 - t0) * 1e3 / args.steps
    if raster:
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step_raster(rev[s])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        rphase = np.mean([[ev[i].elapsed_time(ev[i + 1]) for i in range(2)] for ev in rev], axis=0)
        m["ms_mask"], m["ms_attn"] = (float(x) for x in rphase)
        m["ms_step"] = (t1 - t0) * 1e3 / args.steps
        m["gpu_ms"] = float(rphase.sum())
    else:
        m["ms_mask"], m["ms_attn"], m["ms_step"] = m["ms_mask_x"], m["ms_attn_x"], m["ms_step_x"]
        m["gpu_ms"] = float(phase.sum())
    return m


def loop_step(args, cfg, qd, kd, vd) -> int:
    """The step back to back for args.loop_seconds, a progress line per second (no JSON
    line): a steady load for power and clock readings."""
    step, step_raster, _ = make_steps(cfg, qd, kd, vd)
    main_step = step_raster or step
    for _ in range(max(args.warmup, 1)):
        main_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n, last = 0, t0
    while time.perf_counter() - t0 < args.loop_seconds:
        for _ in range(5):
            main_step()
        torch.cuda.synchronize()
        n += 5
        now = time.perf_counter()
        if now - last >= 1.0:
            say(f"# t={now - t0:.1f}s steps={n} ms/step={(now - t0) * 1e3 / n:.3f}")
            last = now
    return 0


if __name__ == "__main__":
    sys.exit(main())
