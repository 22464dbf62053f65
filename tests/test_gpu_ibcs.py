"""GPU parity of the IBCS block scores (8 query clusters per block scoring the mean keys)
against the oracle.

The oracle clusters in float64 (plain Lloyd's k-means); the kernels cluster in float32.
An assignment whose two nearest centroids are closer than float32 can resolve may go
either way, after which the two clusterings part.  So per query group: where the oracle's
clustering margin (relative gap between the nearest and second-nearest squared distance,
smallest over queries and rounds) is below IBCS_TIE_EPS the group is a near tie, counted
and capped at 2% of groups (at least 2) and left out of the comparison; every other group
must carry the oracle's weights exactly and its centroids within CENT_RTOL.  The scores
are float32 on the GPU (MFMA map, exp2 softmax) and float64 in the oracle: within A_TOL
relative to the row's largest score.  The mask must equal the oracle's CDF cut of its
scores except at the cutoff (the band of the NABLA mask test)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
from synth import Config, get_config, make_qkv
import block_sparse_attention_blockmean_amd as nab
from parity import bitmap_to_mask, check_mask, lists_to_mask

pytestmark = pytest.mark.gpu

K = O.IBCS_CLUSTERS
# float32 logits of size ~10 carry ~1e-6 absolute error, a relative error of ~1e-6 in
# each softmax value; the weighted sum of 8 keeps it there.  20x slack.
A_TOL = 2e-5
# a float32 mean of at most 128 queries, the sum rounded once per query: below
# 128 * 2^-24 ~ 7.6e-6 of the largest coordinate in the worst case (measured ~5e-8)
CENT_RTOL = 8e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, T, H, W, d, dtype, thr, sta=None, heads=2, B=1):
    return Config(name, 12, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=8, N=64, thr=thr,
                  sta=sta, scale_logits=(dtype == "bf16"))


def _up256(n):
    return (n + 255) // 256 * 256


def gpu_ibcs(cfg, qf, kf, thr, sta=None, qn=128):
    """IBCS mask of fractal-ordered GPU tensors with query groups of qn tokens; returns
    lists, bitmap, and the centroids [G, groups, 8, d], weights [G, groups, 8] and score
    rows [G, groups, nb] read back from the workspace."""
    G, nb, d = cfg.BH, cfg.nb, cfg.d
    ng = cfg.L // qn
    nbytes = nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, d, cfg.N, ibcs=True, ibcs_group=qn)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=qf.device)
    cnt, idx, bm = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, sta, with_bitmap=True,
                                  workspace=ws, ibcs=True, ibcs_group=qn)
    torch.cuda.synchronize()
    o_cent = _up256(G * ((nb + 15) // 16 * 16) * d * 4)   # pooled K in tiles of 16 blocks
    o_w = o_cent + _up256(G * ng * K * d * 4)
    o_a = o_w + _up256(G * ng * K * 4)
    assert o_a + _up256(G * ng * nb * 4) == nbytes
    host = ws.cpu()
    cent = host[o_cent:o_cent + G * ng * K * d * 4].view(torch.float32).numpy().reshape(G, ng, K, d)
    w = host[o_w:o_w + G * ng * K * 4].view(torch.float32).numpy().reshape(G, ng, K)
    A = host[o_a:o_a + G * ng * nb * 4].view(torch.float32).numpy().reshape(G, ng, nb)
    # every query block takes its group's row
    A = np.repeat(A, qn // cfg.N, axis=1)
    m = lists_to_mask(cnt.cpu().numpy().reshape(G, nb), idx.cpu().numpy().reshape(G, nb, nb))
    assert np.array_equal(bitmap_to_mask(bm.cpu().numpy().reshape(G, nb, -1), nb), m)
    return dict(cnt=cnt, idx=idx, mask=m, cent=cent, w=w, A=A)


def score_err(gpu_A, ref_A):
    """max over rows of max_j |gpu - oracle| / max_j oracle."""
    ref = np.asarray(ref_A, dtype=np.float64)
    return float(np.max(np.abs(gpu_A - ref).max(-1) / ref.max(-1)))


def check_clusters(res, qf_np, qn, heads):
    """Per query group of the given heads (the oracle clusters all groups of a head at
    once): near-tie groups counted, every other group's weights exactly and centroids
    within CENT_RTOL.  Returns (groups, near-tie groups, per head a [nb] bool of the query
    blocks whose group is a near tie)."""
    ng = res["cent"].shape[1]
    d = qf_np.shape[-1]
    per = qn // 64
    n = n_tie = 0
    tie_rows = []
    for g in heads:
        cent, w, gap = O.ibcs_clusters(qf_np[g, :ng * qn].reshape(ng, qn, d), return_gap=True)
        tie = gap < O.IBCS_TIE_EPS
        ok = ~tie
        gc = res["cent"][g].astype(np.float64)
        assert np.array_equal(res["w"][g][ok].astype(np.float64), w[ok]), (
            f"head {g}: weights of {int((res['w'][g][ok] != w[ok]).any(-1).sum())} groups differ")
        rel = np.max(np.abs(gc - cent), axis=(1, 2)) / np.max(np.abs(cent), axis=(1, 2))
        assert np.all(rel[ok] <= CENT_RTOL), f"head {g}: centroid rel err {rel[ok].max():.3e}"
        n += ng
        n_tie += int(tie.sum())
        tie_rows.append(np.repeat(tie, per))
    assert n_tie <= max(2, int(np.ceil(0.02 * n))), f"{n_tie} of {n} groups are near ties"
    return n, n_tie, np.stack(tie_rows)


def oracle_mask(cfg, qf_np, kf_np, thr, sta=None, qn=128):
    ref = O.ibcs_block_mask(qf_np, kf_np, cfg.N, thr, qn=qn)
    mask = ref["mask"]
    if sta is not None:
        mask = mask | O.sta_mask(cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, sta)[None]
    return mask, ref["A"]


def compare_rows(res_A, res_mask, ref_A, ref_m, tie_rows, thr):
    """Scores within A_TOL and the mask by the band rule on the rows whose group is not a
    near tie; returns (score error, mask mismatches, band population)."""
    keep = ~tie_rows
    err = score_err(res_A[keep], ref_A[keep])
    assert err <= A_TOL, err
    mism, band = check_mask(res_mask[keep], ref_m[keep], ref_A[keep], thr)
    return err, mism, band


CASES = [
    small("bf16_d128_nb75", 5, 24, 40, 128, "bf16", 0.2, heads=1, B=2),
    small("bf16_d64", 3, 32, 16, 64, "bf16", 0.1, heads=3),
    small("bf16_d128_sta", 4, 16, 32, 128, "bf16", 0.3, sta=(3, 3, 3)),
    small("f32_d64", 4, 16, 32, 64, "f32", 0.2),
    small("f32_d128_nb3", 3, 8, 8, 128, "f32", 0.05),
]


@pytest.mark.parametrize("qn", [128, 64])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_ibcs_parity(cfg, qn):
    if cfg.L % qn:
        pytest.skip(f"nb = {cfg.nb} blocks do not split into {qn}-query groups (rejected by the entry point)")
    say(f"IBCS {cfg.name} q_group {qn}: {cfg.B}x{cfg.heads} nb {cfg.nb} d{cfg.d} {cfg.dtype} thr {cfg.thr} "
        f"sta {cfg.sta}")
    q, k, v = make_qkv(cfg)
    G = cfg.BH
    qf = nab.reorder(q.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(k.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    res = gpu_ibcs(cfg, qf, kf, cfg.thr, cfg.sta, qn)
    qnp = qf.float().cpu().numpy().reshape(G, cfg.L, cfg.d)
    knp = kf.float().cpu().numpy().reshape(G, cfg.L, cfg.d)
    n, n_tie, tie_rows = check_clusters(res, qnp, qn, range(G))
    ref_m, ref_A = oracle_mask(cfg, qnp, knp, cfg.thr, cfg.sta, qn)
    err, mism, band = compare_rows(res["A"], res["mask"], ref_A, ref_m, tie_rows, cfg.thr)
    assert np.allclose(res["A"].sum(-1), 1.0, atol=1e-5)
    say(f"  {n} groups ({n_tie} near ties); scores rel err {err:.2e}; kept {res['mask'].mean():.3f}, "
        f"mask mismatches {mism}, band {band}")
    # the top block of every row is kept, as in NABLA
    top = np.argmax(ref_A, axis=-1)
    assert np.all(np.take_along_axis(res["mask"], top[..., None], axis=-1))


@pytest.mark.parametrize("qn", [64, 128])
def test_identical_queries_reduce_to_nabla(qn):
    """When all queries of every group are equal, every query joins cluster 0 (all
    distances tie), its centroid is the query (bf16 values: the running sum is exact)
    and its weight 1, so the IBCS score row is NABLA's pooled softmax row: the lists must
    equal nabla_build_mask's bit for bit."""
    cfg = small("const_blocks", 3, 16, 24, 128, "bf16", 0.2, heads=2)
    q, k, _ = make_qkv(cfg)
    qf = nab.reorder(q.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(k.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    G, nb, N, d = cfg.BH, cfg.nb, cfg.N, cfg.d
    ng = cfg.L // qn
    qc = qf.reshape(G, ng, qn, d)[:, :, :1, :].expand(G, ng, qn, d).reshape(qf.shape).contiguous()
    res = gpu_ibcs(cfg, qc, kf, cfg.thr, qn=qn)
    assert np.all(res["w"][:, :, 0] == 1.0) and np.all(res["w"][:, :, 1:] == 0.0)
    first = qc.float().cpu().numpy().reshape(G, ng, qn, d)[:, :, 0, :]
    assert np.array_equal(res["cent"][:, :, 0, :], first)
    ref = nab.build_mask(qc, kf, cfg.T, cfg.H, cfg.W, cfg.P, N, cfg.thr, with_bitmap=True)
    torch.cuda.synchronize()
    assert torch.equal(ref[0].cpu(), res["cnt"].cpu())
    assert np.array_equal(lists_to_mask(ref[0].cpu().numpy().reshape(G, nb), ref[1].cpu().numpy().reshape(G, nb, nb)),
                          res["mask"])
    say(f"IBCS on constant {qn}-query groups equals the NABLA mask: kept {res['mask'].mean():.3f}")


def test_ibcs_determinism_and_workspace_reuse():
    """Two calls give identical lists; a dirty workspace (left by another call) changes
    nothing."""
    cfg = CASES[1]
    q, k, _ = make_qkv(cfg)
    qf = nab.reorder(q.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(k.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    nbytes = nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, cfg.N, ibcs=True)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")
    a = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, workspace=ws, ibcs=True)
    b = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, ibcs=True)
    torch.cuda.synchronize()
    # only the first kv_count entries of a row are written
    G, nb = cfg.BH, cfg.nb
    assert torch.equal(a[0], b[0])
    ma = lists_to_mask(a[0].cpu().numpy().reshape(G, nb), a[1].cpu().numpy().reshape(G, nb, nb))
    mb = lists_to_mask(b[0].cpu().numpy().reshape(G, nb), b[1].cpu().numpy().reshape(G, nb, nb))
    assert np.array_equal(ma, mb)


@pytest.mark.parametrize("qn", [128, 64])
def test_ibcs_full_size(qn):
    """The Wan-1.3B-like layer at full size: every head through the GPU; centroids of two
    heads bit for bit and their masks against the oracle."""
    cfg = get_config("wan1.3b_480p")
    say(f"IBCS full size {cfg.name} q_group {qn}: {cfg.BH} heads nb {cfg.nb}")
    q, k, _ = make_qkv(cfg)
    G = cfg.BH
    qf = nab.reorder(q.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(k.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    res = gpu_ibcs(cfg, qf, kf, cfg.thr, qn=qn)
    say(f"  GPU mask built: kept {res['mask'].mean():.4f}")
    heads = [0, G - 1]
    qnp = qf.float().cpu().numpy().reshape(G, cfg.L, cfg.d)[heads]
    knp = kf.float().cpu().numpy().reshape(G, cfg.L, cfg.d)[heads]
    sub = dict(cent=res["cent"][heads], w=res["w"][heads])
    n, n_tie, tie_rows = check_clusters(sub, qnp, qn, range(len(heads)))
    ref_m, ref_A = oracle_mask(cfg, qnp, knp, cfg.thr, qn=qn)
    err, mism, band = compare_rows(res["A"][heads], res["mask"][heads], ref_A, ref_m, tie_rows, cfg.thr)
    say(f"  heads {heads}: {n} groups ({n_tie} near ties), scores rel err {err:.2e}, mask mismatches {mism}, "
        f"band {band}")


@pytest.mark.parametrize("qn", [128, 64])
def test_ibcs_max_blocks_per_head(qn):
    """The largest mask the library accepts, 2048 blocks per head (16 frames of 8 x 16
    patches): the score kernel then holds 16 centroid rows of 2048 logits in LDS."""
    cfg = small("nb2048", 16, 64, 128, 64, "bf16", 0.2, heads=1)
    assert cfg.nb == 2048
    say(f"IBCS max blocks per head q_group {qn}: nb {cfg.nb}, L {cfg.L}")
    q, k, _ = make_qkv(cfg)
    qf = nab.reorder(q.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(k.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
    res = gpu_ibcs(cfg, qf, kf, cfg.thr, qn=qn)
    qnp = qf.float().cpu().numpy().reshape(1, cfg.L, cfg.d)
    knp = kf.float().cpu().numpy().reshape(1, cfg.L, cfg.d)
    n, n_tie, tie_rows = check_clusters(res, qnp, qn, [0])
    ref_m, ref_A = oracle_mask(cfg, qnp, knp, cfg.thr, qn=qn)
    err, mism, band = compare_rows(res["A"], res["mask"], ref_A, ref_m, tie_rows, cfg.thr)
    say(f"  {n} groups ({n_tie} near ties); scores rel err {err:.2e}; kept {res['mask'].mean():.4f}, "
        f"mask mismatches {mism}, band {band}")


@pytest.mark.parametrize("qn", [128, 64])
@pytest.mark.parametrize("cfg", [CASES[2], CASES[3]], ids=lambda c: c.name)
def test_ibcs_raster_equals_explicit_reorder(cfg, qn):
    """nabla_build_mask_ibcs_raster on raster-order Q, K gives the lists, bitmap and
    workspace (pooled K, centroids, weights, scores) of nabla_reorder followed by
    nabla_build_mask_ibcs, bit for bit."""
    q, k, _ = make_qkv(cfg)
    qd, kd = q.cuda(), k.cuda()
    qf = nab.reorder(qd, cfg.T, cfg.H, cfg.W, cfg.P)
    kf = nab.reorder(kd, cfg.T, cfg.H, cfg.W, cfg.P)
    nbytes = nab.build_mask_workspace_size(cfg.B, cfg.heads, cfg.L, cfg.d, cfg.N, ibcs=True, ibcs_group=qn)
    ws_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, cfg.sta, with_bitmap=True,
                       with_schedule=True, workspace=ws_a, ibcs=True, ibcs_group=qn)
    b = nab.build_mask(qd, kd, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr, cfg.sta, with_bitmap=True,
                       with_schedule=True, workspace=ws_b, ibcs=True, ibcs_group=qn, raster=True)
    torch.cuda.synchronize()
    G, nb = cfg.BH, cfg.nb
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])
    ma = lists_to_mask(a[0].cpu().numpy().reshape(G, nb), a[1].cpu().numpy().reshape(G, nb, nb))
    mb = lists_to_mask(b[0].cpu().numpy().reshape(G, nb), b[1].cpu().numpy().reshape(G, nb, nb))
    assert np.array_equal(ma, mb)
    assert torch.equal(ws_a, ws_b), "workspace sections differ"
    say(f"IBCS raster == explicit reorder, {cfg.name} q_group {qn}: kept {ma.mean():.3f}")
