"""GPU parity of the SIP selection (sampled blocks with Horvitz-Thompson logit shifts)
and of the weighted attention against the oracle.

Keep decisions must match the oracle's except where the draw lies within 1e-5 of the
oracle's inclusion probability (the probabilities carry the float32 error of the pooled
map); log-weights of blocks kept on both sides within 1e-4; attention within the usual
1e-4 (float32) / 2e-2 (bf16) of the oracle run on the GPU's own lists and weights."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
from synth import Config, get_config, make_qkv
import block_sparse_attention_blockmean_amd as nab
from parity import TOL_BF16, TOL_F32, lists_to_mask, max_abs

pytestmark = pytest.mark.gpu

U_BAND = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, T, H, W, d, dtype, heads=2, B=1):
    return Config(name, 6, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=8, N=64, thr=0.2,
                  sta=None, scale_logits=(dtype == "bf16"))


def gpu_sip(cfg, q, k, budget, seed):
    G, nb = cfg.BH, cfg.nb
    u = torch.rand((cfg.B, cfg.heads, nb, nb), generator=torch.Generator().manual_seed(seed))
    qd, kd = q.cuda(), k.cuda()
    qf, kf = (nab.reorder(t, cfg.T, cfg.H, cfg.W, cfg.P) for t in (qd, kd))
    cnt, idx, logw, bm = nab.build_mask_sip(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, budget, u.cuda(),
                                            cfg.N, with_bitmap=True)
    torch.cuda.synchronize()
    cn = cnt.cpu().numpy().reshape(G, nb)
    ix = idx.cpu().numpy().reshape(G, nb, nb)
    lw = logw.cpu().numpy().reshape(G, nb, nb)
    m = lists_to_mask(cn, ix)
    # dense [G, nb, nb] log-weights from the lists
    dense_w = np.zeros((G, nb, nb))
    for g in range(G):
        for i in range(nb):
            dense_w[g, i, ix[g, i, :cn[g, i]]] = lw[g, i, :cn[g, i]]
    return dict(qf=qf, kf=kf, cnt=cnt, idx=idx, logw=logw, bitmap=bm, mask=m, dense_w=dense_w,
                u=u.numpy().reshape(G, nb, nb))


def oracle_sip(cfg, q, k, budget, u):
    G = cfg.BH
    qn, kn = (t.float().numpy().reshape(G, cfg.L, cfg.d) for t in (q, k))
    qf, kf = (O.reorder(a, cfg.T, cfg.H, cfg.W, cfg.P) for a in (qn, kn))
    A = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, 0.0)["A"]
    m, logw, pi = O.sip_mask(A, budget, u)
    return m, logw, pi


def check_sip(res, ref_m, ref_w, ref_pi, budget):
    m, u = res["mask"], res["u"]
    mism = m != ref_m
    near = np.abs(u - ref_pi) <= U_BAND
    assert not (mism & ~near).any(), f"{int((mism & ~near).sum())} keep decisions differ away from the band"
    both = m & ref_m
    err_w = float(np.max(np.abs(res["dense_w"][both] - ref_w[both]))) if both.any() else 0.0
    assert err_w <= 1e-4, err_w
    assert np.all(res["cnt"].cpu().numpy() >= 1), "the top block of every row is kept"
    return int(mism.sum()), err_w


SMALL = [
    small("bf16_d128", 5, 24, 40, 128, "bf16", heads=1, B=2),
    small("bf16_d64", 3, 32, 16, 64, "bf16", heads=3),
    small("f32_d64", 4, 16, 32, 64, "f32"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_sip_parity(cfg):
    q, k, v = make_qkv(cfg)
    nb = cfg.nb
    for budget in (1, 2, max(2, nb // 6), nb // 2, nb):
        res = gpu_sip(cfg, q, k, budget, seed=budget + 7)
        ref_m, ref_w, ref_pi = oracle_sip(cfg, q, k, budget, res["u"])
        mism, err_w = check_sip(res, ref_m, ref_w, ref_pi, budget)
        kept = res["mask"].sum(-1).mean()
        say(f"{cfg.name} budget {budget}: mean kept {kept:.2f} (expected {min(budget, nb)}), "
            f"band mismatches {mism}, logw err {err_w:.2e}")
        if budget >= nb:
            assert res["mask"].all() and np.all(res["dense_w"] == 0)
        # weighted attention with the GPU's own lists and weights
        G = cfg.BH
        vf = nab.reorder(v.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
        o = nab.attn_fwd_weighted(res["qf"], res["kf"], vf, res["cnt"], res["idx"], res["logw"], cfg.N)
        torch.cuda.synchronize()
        args = [t.float().cpu().numpy().reshape(G, cfg.L, cfg.d) for t in (res["qf"], res["kf"], vf)]
        ref_o = O.weighted_block_attention(*args, res["mask"], res["dense_w"], cfg.N)
        err = max_abs(o.float().cpu().numpy().reshape(G, cfg.L, cfg.d), ref_o)
        tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
        say(f"  weighted attention max-abs {err:.3e} (tol {tol})")
        assert err <= tol
        if budget >= nb:
            plain = nab.attn_fwd(res["qf"], res["kf"], vf, res["cnt"], res["idx"], cfg.N)
            torch.cuda.synchronize()
            assert torch.equal(plain, o), "zero shifts must give the unweighted kernel's bits"


def test_sip_full_size():
    """The Wan-1.3B-like layer with the NABLA run's average kept count as the budget:
    decisions and weights of two heads against the oracle, and the expected budget."""
    cfg = get_config("wan1.3b_480p")
    q, k, v = make_qkv(cfg)
    budget = 185
    res = gpu_sip(cfg, q, k, budget, seed=99)
    G, nb = cfg.BH, cfg.nb
    kept = res["mask"].sum(-1)
    say(f"full size SIP budget {budget}: mean kept {kept.mean():.2f}")
    # the kept count of a row is a sum of independent Bernoulli(pi_j): its mean over the
    # 6048 rows is within a few standard errors of the budget
    assert abs(kept.mean() - budget) <= 2.0
    for g in (0, G - 1):
        sl = slice(g, g + 1)
        qn, kn = (t.float().numpy().reshape(G, cfg.L, cfg.d)[sl] for t in (q, k))
        qf, kf = (O.reorder(a, cfg.T, cfg.H, cfg.W, cfg.P) for a in (qn, kn))
        A = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, 0.0)["A"]
        ref_m, ref_w, ref_pi = O.sip_mask(A, budget, res["u"][sl])
        sub = dict(mask=res["mask"][sl], u=res["u"][sl], dense_w=res["dense_w"][sl], cnt=res["cnt"].reshape(G, nb)[sl])
        mism, err_w = check_sip(sub, ref_m, ref_w, ref_pi, budget)
        say(f"  head {g}: band mismatches {mism}, logw err {err_w:.2e}")


@pytest.mark.parametrize("qn", [128, 64])
@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2]], ids=lambda c: c.name)
def test_ibcs_sip_parity(cfg, qn):
    """The AB-Attention page's selectors together: SIP sampling from IBCS scores
    (q_group-query clusters).  Decisions against the oracle's sip_mask of its
    ibcs_scores, within the draw band; log-weights; weighted attention on the GPU's
    lists."""
    q, k, v = make_qkv(cfg)
    G, nb = cfg.BH, cfg.nb
    qd, kd = q.cuda(), k.cuda()
    qf, kf = (nab.reorder(t, cfg.T, cfg.H, cfg.W, cfg.P) for t in (qd, kd))
    qnp, knp = (t.float().cpu().numpy().reshape(G, cfg.L, cfg.d) for t in (qf, kf))
    A, gap = O.ibcs_scores(qnp, knp, cfg.N, qn=qn, return_gap=True)
    # rows whose query group is a float32 near tie of the clustering are left out (see
    # test_gpu_ibcs.py); at most 2% of groups, at least 2
    keep = gap >= O.IBCS_TIE_EPS
    assert (~keep).sum() <= max(2, int(np.ceil(0.02 * keep.size))) * (qn // cfg.N)
    for budget in (1, max(2, nb // 6), nb // 2, nb):
        u = torch.rand((cfg.B, cfg.heads, nb, nb), generator=torch.Generator().manual_seed(budget + 100))
        cnt, idx, logw, bm = nab.build_mask_sip(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, budget, u.cuda(), cfg.N,
                                                with_bitmap=True, ibcs=True, ibcs_group=qn)
        torch.cuda.synchronize()
        cn = cnt.cpu().numpy().reshape(G, nb)
        ix = idx.cpu().numpy().reshape(G, nb, nb)
        lw = logw.cpu().numpy().reshape(G, nb, nb)
        m = lists_to_mask(cn, ix)
        dense_w = np.zeros((G, nb, nb))
        for g in range(G):
            for i in range(nb):
                dense_w[g, i, ix[g, i, :cn[g, i]]] = lw[g, i, :cn[g, i]]
        un = u.numpy().reshape(G, nb, nb)
        ref_m, ref_w, ref_pi = O.sip_mask(A, budget, un)
        res = dict(mask=m[keep], u=un[keep], dense_w=dense_w[keep], cnt=cnt.reshape(G, nb)[torch.from_numpy(keep).cuda()])
        mism, err_w = check_sip(res, ref_m[keep], ref_w[keep], ref_pi[keep], budget)
        say(f"IBCS+SIP {cfg.name} q_group {qn} budget {budget}: mean kept {m.sum(-1).mean():.2f}, "
            f"band mismatches {mism}, logw err {err_w:.2e}")
        vf = nab.reorder(v.cuda(), cfg.T, cfg.H, cfg.W, cfg.P)
        o = nab.attn_fwd_weighted(qf, kf, vf, cnt, idx, logw, cfg.N)
        torch.cuda.synchronize()
        args = [t.float().cpu().numpy().reshape(G, cfg.L, cfg.d) for t in (qf, kf, vf)]
        ref_o = O.weighted_block_attention(*args, m, dense_w, cfg.N)
        err = max_abs(o.float().cpu().numpy().reshape(G, cfg.L, cfg.d), ref_o)
        tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
        assert err <= tol, err
