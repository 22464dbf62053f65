"""GPU parity: every step of the HIP path against the oracle on the same seeded inputs.

Masks must match bit for bit except blocks whose oracle cumulative mass lies within
1e-4 of thr (at most 0.1% of blocks); outputs must match the oracle evaluated with the
GPU's own mask within 1e-4 (float32) / 2e-2 (bf16) max-abs.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, Config, get_config, make_head, make_qkv
import block_sparse_attention_blockmean_amd as nab
from parity import (TOL_BF16, TOL_F32, bitmap_to_mask, check_mask, lists_to_mask, max_abs)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def tdtype(cfg: Config):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def small(name, T, H, W, P, d, dtype, thr, sta=None, heads=2, B=1, seed_index=7):
    return Config(name, seed_index, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=P,
                  N=64, thr=thr, sta=sta, scale_logits=(dtype == "bf16"))


SMALL = [
    get_config("tiny"),
    dataclasses.replace(get_config("tiny"), name="tiny_thr0", thr=0.0),
    dataclasses.replace(get_config("tiny"), name="tiny_thr05", thr=0.5),
    small("bf16_d128_ragged", 5, 24, 40, 8, 128, "bf16", 0.2),
    small("bf16_d128_ragged_sta", 5, 24, 40, 8, 128, "bf16", 0.2, sta=(3, 3, 3)),
    small("bf16_d64", 3, 32, 32, 8, 64, "bf16", 0.05, heads=3),
    small("bf16_P4", 2, 16, 16, 4, 128, "bf16", 0.1),
    small("f32_d128_sta", 4, 16, 32, 8, 128, "f32", 0.3, sta=(1, 3, 5)),
    small("bf16_nb130", 13, 16, 40, 8, 128, "bf16", 0.2, B=2, heads=1),
]


def run_gpu_path(cfg: Config, q, k, v, thr=None, with_bitmap=True):
    """Raster CPU tensors -> GPU reorder, mask, attention, inverse reorder."""
    thr = cfg.thr if thr is None else thr
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qf = nab.reorder(qd, cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(kd, cfg.T, cfg.H, cfg.W, cfg.P)
    vf = nab.reorder(vd, cfg.T, cfg.H, cfg.W, cfg.P)
    cnt, idx, bm, sched = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, cfg.sta,
                                         with_bitmap=True, with_schedule=True)
    of = nab.attn_fwd(qf, kf, vf, cnt, idx, cfg.N, schedule=sched)
    o = nab.reorder(of, cfg.T, cfg.H, cfg.W, cfg.P, inverse=True)
    torch.cuda.synchronize()
    return dict(qf=qf, kf=kf, vf=vf, cnt=cnt, idx=idx, bitmap=bm, sched=sched, of=of, o=o)


# ------------------------------------------------------------------ reorder

@pytest.mark.parametrize("T,H,W,P,d,dt", [
    (4, 16, 16, 8, 64, torch.float32), (3, 24, 40, 8, 128, torch.bfloat16),
    (2, 12, 20, 4, 64, torch.bfloat16), (2, 8, 8, 1, 128, torch.float32),
    (1, 16, 16, 16, 64, torch.bfloat16), (5, 6, 9, 3, 64, torch.float32),
])
def test_reorder_bitexact(T, H, W, P, d, dt):
    say(f"reorder T{T} H{H} W{W} P{P} d{d} {dt}")
    g = torch.Generator().manual_seed(T * 1000 + H * 10 + P)
    x = torch.randn(2, 3, T * H * W, d, generator=g).to(dt)
    y = nab.reorder(x.cuda(), T, H, W, P)
    z = nab.reorder(y, T, H, W, P, inverse=True)
    ref = O.reorder(x.view(torch.int16 if dt == torch.bfloat16 else torch.int32).numpy(), T, H, W, P)
    yb = y.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(yb, ref)
    assert torch.equal(z.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       x.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


# ------------------------------------------------------------------ mask + attention, small grids

@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_grid_parity(cfg):
    say(f"small-grid parity {cfg.name}: {cfg.B}x{cfg.heads} {cfg.T}x{cfg.H}x{cfg.W} P{cfg.P} "
        f"d{cfg.d} {cfg.dtype} thr{cfg.thr} sta{cfg.sta} nb{cfg.nb}")
    q, k, v = make_qkv(cfg)
    res = run_gpu_path(cfg, q, k, v)
    G = cfg.BH
    qn, kn, vn = (to_np(t).reshape(G, cfg.L, cfg.d) for t in (q, k, v))
    qf, kf, vf = (O.reorder(a, cfg.T, cfg.H, cfg.W, cfg.P) for a in (qn, kn, vn))
    # the GPU reorder is exact, so the fractal tensors agree bit for bit
    assert np.array_equal(to_np(res["qf"]).reshape(G, cfg.L, cfg.d), qf)
    ref = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, cfg.sta)
    cnt = res["cnt"].cpu().numpy().reshape(G, cfg.nb)
    idx = res["idx"].cpu().numpy().reshape(G, cfg.nb, cfg.nb)
    gmask = lists_to_mask(cnt, idx)
    assert np.array_equal(bitmap_to_mask(res["bitmap"].cpu().numpy().reshape(G, cfg.nb, -1), cfg.nb),
                          gmask)
    mism, band = check_mask(gmask, ref["mask"], ref["A"], cfg.thr)
    assert np.all(cnt >= 1), "the largest block of every row is kept"
    say(f"  kept {gmask.mean():.4f}  mismatches {mism}  band {band}")
    # attention with the GPU's own mask
    out = O.masked_attention(qf, kf, vf, gmask, cfg.N)
    err = max_abs(to_np(res["of"]).reshape(G, cfg.L, cfg.d), out)
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    say(f"  attention max-abs {err:.3e} (tol {tol})")
    assert err <= tol
    # the whole path, back in raster order
    err_r = max_abs(to_np(res["o"]).reshape(G, cfg.L, cfg.d),
                    O.reorder(out, cfg.T, cfg.H, cfg.W, cfg.P, inverse=True))
    assert err_r <= tol


def test_thr0_is_full_attention():
    """thr = 0 keeps every block, so the path is dense attention in raster order."""
    cfg = dataclasses.replace(get_config("tiny"), thr=0.0)
    q, k, v = make_qkv(cfg)
    res = run_gpu_path(cfg, q, k, v)
    assert torch.all(res["cnt"] == cfg.nb)
    qt, kt, vt = (t.double() for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()
    assert max_abs(to_np(res["o"]), ref) <= TOL_F32


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_attention_arbitrary_lists(dtype, d):
    """Lists not produced by the mask step: random rows, full rows and empty rows."""
    cfg = small("lists", 3, 16, 24, 8, d, dtype, 0.1, heads=2)
    say(f"arbitrary lists {dtype} d{d}")
    q, k, v = make_qkv(cfg)
    G, nb = cfg.BH, cfg.nb
    rng = np.random.default_rng(5)
    m = rng.random((G, nb, nb)) < 0.3
    m[:, 0, :] = True          # a full row
    m[:, 1, :] = False         # an empty row -> zeros
    m[:, 2, :] = False
    m[:, 2, nb - 1] = True     # a single far block
    cnt, idx = O.kv_lists(m)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = nab.attn_fwd(qd, kd, vd, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ref = O.masked_attention(*(to_np(t).reshape(G, cfg.L, d) for t in (q, k, v)), m, cfg.N)
    on = to_np(o).reshape(G, cfg.L, d)
    assert np.all(on[:, 64:128] == 0)
    assert max_abs(on, ref) <= (TOL_BF16 if dtype == "bf16" else TOL_F32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_ties_grouped(dtype):
    """Blocks with identical keys get identical pooled probabilities on both sides;
    tied blocks must be kept or dropped together, and with exact ties the plain
    |F - thr| <= 1e-4 band applies."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(11)
    L, d, N = 1024, 64, 64
    q = torch.randn(1, 2, L, d, generator=g).to(tdt)
    k = torch.randn(1, 2, L, d, generator=g).to(tdt) * 2
    # 16 key blocks made of 4 distinct blocks, each repeated 4 times
    kb = k.reshape(1, 2, 16, N, d)
    for j in range(4, 16):
        kb[:, :, j] = kb[:, :, j % 4]
    k = kb.reshape(1, 2, L, d).contiguous()
    qn = to_np(q).reshape(2, L, d)
    kn = to_np(k).reshape(2, L, d)
    for thr in (0.05, 0.2, 0.3, 0.45, 0.6, 0.8):
        cnt, idx = nab.build_mask(q.cuda(), k.cuda(), 4, 16, 16, 8, N, thr)
        torch.cuda.synchronize()
        gm = lists_to_mask(cnt.cpu().numpy().reshape(2, 16), idx.cpu().numpy().reshape(2, 16, 16))
        for j in range(4, 16):
            assert np.array_equal(gm[..., j], gm[..., j % 4]), (thr, j)
        ref = O.block_mask(qn, kn, 4, 16, 16, 8, N, thr)
        mism = gm != ref["mask"]
        assert np.all(np.abs(ref["F"][mism] - thr) <= 1e-4), thr


def check_pair_schedule(cfg, sched, cnt):
    """The mask step's start order: a permutation of the query blocks in which entries 2j
    and 2j + 1 form a pair - block i of frame t with block i of frame t + 1 (t even), the
    last frame's blocks side by side when the frame count is odd - heads in order, each
    head's pairs by non-increasing combined kept count, and the one block per head left
    without a partner (odd frame count and odd blocks per frame) at the very end."""
    G, nb = cfg.BH, cfg.nb
    assert np.array_equal(np.sort(sched), np.arange(G * nb))
    fpf = cfg.H * cfg.W // cfg.N if (cfg.H * cfg.W) % cfg.N == 0 else 1
    frames = nb // fpf
    single = (frames % 2) * (fpf % 2)
    for g in range(G):
        part = sched[g * (nb - single):(g + 1) * (nb - single)]
        assert np.all(part // nb == g), "a head's pairs stay in its region"
        a, b = part[0::2] - g * nb, part[1::2] - g * nb
        temporal = (b == a + fpf) & ((a // fpf) % 2 == 0)
        last = (a // fpf == frames - 1) & (b == a + 1) & ((a % fpf) % 2 == 0)
        assert np.all(temporal | (last & (frames % 2 == 1))), "pairs are neighbours in time"
        sums = cnt[g * nb + a] + cnt[g * nb + b]
        assert np.all(np.diff(sums) <= 0), "pairs by non-increasing combined count"
    if single:
        assert np.array_equal(sched[G * (nb - 1):], np.arange(G) * nb + nb - 1)


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[3], SMALL[8]], ids=lambda c: c.name)
def test_schedule(cfg):
    """The start order pairs neighbouring frames' blocks, and the attention output does not
    depend on the order or the pairing: reversed, shuffled (pairs across heads) and no
    order at all give the same bits."""
    q, k, v = make_qkv(cfg)
    res = run_gpu_path(cfg, q, k, v)
    sched = res["sched"].cpu().numpy()
    cnt = res["cnt"].cpu().numpy().reshape(-1)
    check_pair_schedule(cfg, sched, cnt)
    plain = nab.attn_fwd(res["qf"], res["kf"], res["vf"], res["cnt"], res["idx"], cfg.N)
    rev = torch.flip(res["sched"], [0]).contiguous()
    backwards = nab.attn_fwd(res["qf"], res["kf"], res["vf"], res["cnt"], res["idx"], cfg.N,
                             schedule=rev)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(cfg.BH * cfg.nb).astype(np.int32)).cuda()
    shuffled = nab.attn_fwd(res["qf"], res["kf"], res["vf"], res["cnt"], res["idx"], cfg.N, schedule=perm)
    torch.cuda.synchronize()
    assert torch.equal(plain, res["of"])
    assert torch.equal(backwards, res["of"])
    assert torch.equal(shuffled, res["of"])


def test_determinism():
    """Repeated runs give identical bits (no atomics or order-dependent reductions)."""
    cfg = SMALL[4]
    q, k, v = make_qkv(cfg)
    a = run_gpu_path(cfg, q, k, v)
    b = run_gpu_path(cfg, q, k, v)
    assert torch.equal(a["cnt"], b["cnt"])
    for key in ("bitmap", "o"):
        assert torch.equal(a[key], b[key])


# ------------------------------------------------------------------ full-size workloads

def _sample_blocks(G, nb, cnt, rng, n_rand=48):
    pairs = {(0, 0), (0, nb - 1), (G - 1, 0), (G - 1, nb - 1)}
    flat = cnt.reshape(-1)
    for f in (int(np.argmax(flat)), int(np.argmin(flat))):
        pairs.add((f // nb, f % nb))
    for _ in range(n_rand):
        pairs.add((int(rng.integers(G)), int(rng.integers(nb))))
    return sorted(pairs)


def test_max_blocks_per_head():
    """The largest mask the library accepts: 2048 blocks per head (16 frames of 8 x 16
    patches), where the select step holds 16 rows of 2048 pooled logits in LDS."""
    cfg = small("nb2048", 16, 64, 128, 8, 64, "bf16", 0.2, heads=1)
    assert cfg.nb == 2048
    say(f"max blocks per head: nb {cfg.nb}, L {cfg.L}")
    q, k, v = make_qkv(cfg)
    res = run_gpu_path(cfg, q, k, v)
    nb = cfg.nb
    cnt = res["cnt"].cpu().numpy().reshape(1, nb)
    idx = res["idx"].cpu().numpy().reshape(1, nb, nb)
    gmask = lists_to_mask(cnt, idx)
    assert np.array_equal(bitmap_to_mask(res["bitmap"].cpu().numpy().reshape(1, nb, -1), nb), gmask)
    qf, kf, vf = (O.reorder(to_np(t.reshape(1, cfg.L, cfg.d)[0]), cfg.T, cfg.H, cfg.W, cfg.P)
                  for t in (q, k, v))
    ref = O.block_mask(qf[None], kf[None], cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr)
    mism, band = check_mask(gmask, ref["mask"], ref["A"], cfg.thr)
    say(f"  kept {gmask.mean():.4f}  mismatches {mism}  band {band}")
    assert mism <= 1e-3 * gmask.size
    of = res["of"].reshape(1, cfg.L, cfg.d)
    worst = 0.0
    for _, i in _sample_blocks(1, nb, cnt, np.random.default_rng(11), n_rand=12):
        ref_o = O.attention_block(qf, kf, vf, gmask[0, i], i, cfg.N, 1.0 / np.sqrt(cfg.d))
        worst = max(worst, max_abs(to_np(of[0, i * cfg.N:(i + 1) * cfg.N]), ref_o))
    say(f"  attention on sampled blocks: max-abs {worst:.3e}")
    assert worst <= TOL_BF16


def _full_sample(G, nb, cnt, rng, frac=0.05):
    """Every query block of the first and the last (batch, head), plus a seeded 5%
    of the blocks of every other head (at least one per head), plus the longest and the
    shortest list."""
    pairs = {(g, i) for g in {0, G - 1} for i in range(nb)}
    per = max(1, int(round(frac * nb)))
    for g in range(1, G - 1):
        for i in rng.choice(nb, size=per, replace=False):
            pairs.add((g, int(i)))
    flat = cnt.reshape(-1)
    for f in (int(np.argmax(flat)), int(np.argmin(flat))):
        pairs.add((f // nb, f % nb))
    return sorted(pairs)


def _raster_path(cfg, qd, kd, vd, thr, sta):
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    cnt, idx, bm, sched = nab.build_mask(qd, kd, T, H, W, P, N, thr, sta, with_bitmap=True, with_schedule=True,
                                         raster=True)
    o = nab.attn_fwd_raster(qd, kd, vd, cnt, idx, T, H, W, P, N, schedule=sched)
    torch.cuda.synchronize()
    return cnt, idx, bm, sched, o


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [c for c in CONFIGS if c.name != "tiny"], ids=lambda c: c.name)
def test_full_config_parity(cfg):
    """At full size, for every threshold of the workload: the raster-order entry points
    (the path the bench times) give the explicit path's counts, lists, bitmap, start order
    and output bit for bit; the mask matches the oracle on every head by the band rule,
    with its mismatches split into plain-band and near-tie-only ones; with a window, the
    window-free mask (STA off) matches the oracle's CDF part on its own, and the kept
    fractions of the CDF part, the window and their union are reported; attention matches
    the oracle (evaluated with the GPU's mask, float32) on every query block of the first
    and last (batch, head) and a seeded 5% of the others' (rows are independent given the
    mask, so each is an exact check)."""
    say(f"full config {cfg.name}: {cfg.B}x{cfg.heads} L{cfg.L} nb{cfg.nb}")
    q, k, v = make_qkv(cfg)
    say("  inputs generated")
    G, nb = cfg.BH, cfg.nb
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    sta_part = None
    if cfg.sta is not None:
        sta_part = O.sta_mask(cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.sta)
    for thr in (cfg.thr_list or (cfg.thr,)):
        res = run_gpu_path(cfg, q, k, v, thr=thr)
        ras = _raster_path(cfg, qd, kd, vd, thr, cfg.sta)
        assert torch.equal(res["cnt"], ras[0]) and torch.equal(res["bitmap"], ras[2])
        assert torch.equal(res["sched"], ras[3])
        assert torch.equal(res["o"].view(torch.int16), ras[4].view(torch.int16)), "raster output differs"
        cnt = res["cnt"].cpu().numpy().reshape(G, nb)
        idx = res["idx"].cpu().numpy().reshape(G, nb, nb)
        gmask = lists_to_mask(cnt, idx)
        assert np.array_equal(lists_to_mask(cnt, ras[1].cpu().numpy().reshape(G, nb, nb)), gmask)
        del ras
        # the window-free mask of the same inputs (the CDF part alone)
        nabla_only = None
        if cfg.sta is not None:
            c2, i2 = nab.build_mask(res["qf"], res["kf"], cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, None)
            torch.cuda.synchronize()
            nabla_only = lists_to_mask(c2.cpu().numpy().reshape(G, nb), i2.cpu().numpy().reshape(G, nb, nb))
            assert np.all(gmask >= nabla_only) and np.all(gmask >= sta_part[None])
            assert np.array_equal(gmask, nabla_only | sta_part[None])
        counts, counts_nabla = {}, {}
        # oracle mask, a few heads at a time to bound host memory
        for g0 in range(0, G, 8):
            sl = slice(g0, min(G, g0 + 8))
            qn = to_np(q.reshape(G, cfg.L, cfg.d)[sl])
            kn = to_np(k.reshape(G, cfg.L, cfg.d)[sl])
            qf = O.reorder(qn, cfg.T, cfg.H, cfg.W, cfg.P)
            kf = O.reorder(kn, cfg.T, cfg.H, cfg.W, cfg.P)
            ref = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, cfg.sta)
            check_mask(gmask[sl], ref["mask"], ref["A"], thr, ref["F"], counts)
            if nabla_only is not None:
                check_mask(nabla_only[sl], ref["mask_nabla"], ref["A"], thr, ref["F"], counts_nabla)
        say(f"  thr {thr}: kept {gmask.mean():.4f}; mask mismatches {counts['mismatches']} of {counts['blocks']} "
            f"(plain band {counts['plain']}, near-tie only {counts['tie_only']}), band population {counts['band']}")
        if nabla_only is not None:
            say(f"  thr {thr}: kept fractions: CDF part {nabla_only.mean():.4f}, window {sta_part.mean():.4f}, "
                f"union {gmask.mean():.4f}; CDF-part mismatches {counts_nabla['mismatches']} "
                f"(plain band {counts_nabla['plain']}, near-tie only {counts_nabla['tie_only']})")
        rng = np.random.default_rng(cfg.index)
        blocks = _full_sample(G, nb, cnt, rng)
        of = res["of"].reshape(G, cfg.L, cfg.d)
        worst = 0.0
        heads = sorted({g for g, _ in blocks})
        for g in heads:
            qf, kf, vf = (O.reorder(to_np(t.reshape(G, cfg.L, cfg.d)[g]), cfg.T, cfg.H, cfg.W, cfg.P)
                          for t in (q, k, v))
            got_h = to_np(of[g])
            for gg, i in blocks:
                if gg != g:
                    continue
                ref_o = O.attention_block(qf, kf, vf, gmask[g, i], i, cfg.N, 1.0 / np.sqrt(cfg.d), np.float32)
                worst = max(worst, max_abs(got_h[i * cfg.N:(i + 1) * cfg.N], ref_o))
        say(f"  attention on {len(blocks)} query blocks ({len(heads)} heads): max-abs {worst:.3e}")
        assert worst <= TOL_BF16
        del res
        torch.cuda.empty_cache()


LONG = [
    small("bf16_nb1500", 25, 48, 80, 8, 128, "bf16", 0.2, heads=3, seed_index=13),
    small("f32_d64_nb1980_sta", 33, 48, 80, 8, 64, "f32", 0.1, sta=(3, 3, 3), heads=1, seed_index=14),
    small("bf16_nb2400_sta", 40, 48, 80, 8, 128, "bf16", 0.2, sta=(3, 3, 3), seed_index=11),
    small("bf16_nb4080", 68, 48, 80, 8, 128, "bf16", 0.1, heads=1, seed_index=12),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", LONG, ids=lambda c: c.name)
def test_long_rows(cfg):
    """Long rows: 1,500 and 1,980 blocks (24 and 32 registers per lane, two rows per wave in
    the map kernel) and beyond 2048 blocks (48 and 64 registers, up to the 4096-block
    limit): explicit and raster paths bit-equal, the mask against the oracle by the band
    rule on every head, attention on a seeded sample of query blocks."""
    say(f"long rows {cfg.name}: {cfg.B}x{cfg.heads} nb{cfg.nb}")
    q, k, v = make_qkv(cfg)
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    G, nb = cfg.BH, cfg.nb
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    res = run_gpu_path(cfg, q, k, v)
    ras = _raster_path(cfg, qd, kd, vd, cfg.thr, cfg.sta)
    assert torch.equal(res["cnt"], ras[0]) and torch.equal(res["bitmap"], ras[2])
    assert torch.equal(res["sched"], ras[3])
    bits = (lambda t: t.view(torch.int16)) if cfg.dtype == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(res["o"]), bits(ras[4]))
    cnt = res["cnt"].cpu().numpy().reshape(G, nb)
    gmask = lists_to_mask(cnt, res["idx"].cpu().numpy().reshape(G, nb, nb))
    check_pair_schedule(cfg, res["sched"].cpu().numpy(), cnt.reshape(-1))
    counts = {}
    rng = np.random.default_rng(cfg.index)
    worst = 0.0
    for g in range(G):
        qf, kf, vf = (O.reorder(to_np(t.reshape(G, cfg.L, cfg.d)[g]), cfg.T, cfg.H, cfg.W, cfg.P) for t in (q, k, v))
        ref = O.block_mask(qf[None], kf[None], cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, cfg.sta)
        check_mask(gmask[g:g + 1], ref["mask"], ref["A"], cfg.thr, ref["F"], counts)
        got = to_np(res["of"].reshape(G, cfg.L, cfg.d)[g])
        for i in sorted({0, nb - 1, *rng.choice(nb, size=16, replace=False).tolist()}):
            ref_o = O.attention_block(qf, kf, vf, gmask[g, i], i, cfg.N, 1.0 / np.sqrt(cfg.d), np.float32)
            worst = max(worst, max_abs(got[i * cfg.N:(i + 1) * cfg.N], ref_o))
    say(f"  kept {gmask.mean():.4f}; mask mismatches {counts['mismatches']} of {counts['blocks']} "
        f"(plain band {counts['plain']}, near-tie only {counts['tie_only']}); attention max-abs {worst:.3e}")
    assert worst <= tol
