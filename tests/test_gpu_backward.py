"""GPU parity of the attention gradient (and of the forward's log-sum-exp) against the
oracle on the same seeded inputs.

Gradients are compared with the oracle's float64 gradient of the masked attention on
the same (bf16-rounded) inputs and the same lists, scaled by the size of each gradient:
max |gpu - oracle| <= tol * max(1, max |oracle|), tol = 2e-2 (bf16) / 1e-4 (float32).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
from synth import Config, get_config, make_qkv
import block_sparse_attention_blockmean_amd as nab
from parity import lists_to_mask, max_abs

pytestmark = pytest.mark.gpu

TOL_GRAD = {"bf16": 2e-2, "f32": 1e-4}
TOL_LSE = {"bf16": 1e-3, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def small(name, T, H, W, d, dtype, heads=2, B=1, seed_index=9):
    return Config(name, seed_index, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=8,
                  N=64, thr=0.2, sta=None, scale_logits=(dtype == "bf16"))


def random_lists(G, nb, rng, density=0.3):
    m = rng.random((G, nb, nb)) < density
    m[:, np.arange(nb), np.arange(nb)] = True
    m[:, 0, :] = True            # a full row
    m[:, 1, :] = False           # an empty row: zero output, no gradient
    m[:, 2, :] = False
    m[:, 2, nb - 1] = True       # a single far block
    m[:, :, 3] = False           # a KV block no row keeps: zero dK, dV
    return m


def grad_err(gpu, ref):
    scale = max(1.0, float(np.max(np.abs(ref))))
    return max_abs(gpu, ref) / scale


def run_fwd_bwd(q, k, v, dout, cnt, idx, N=64):
    o, lse = nab.attn_fwd(q, k, v, cnt, idx, N, with_lse=True)
    dq, dk, dv = nab.attn_bwd(q, k, v, o, dout, lse, cnt, idx, N)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


CASES = [
    small("bf16_d128", 3, 16, 24, 128, "bf16"),
    small("bf16_d64", 2, 24, 32, 64, "bf16", heads=3),
    small("bf16_d128_nb75", 5, 24, 40, 128, "bf16", heads=1, B=2),
    small("f32_d64", 2, 16, 16, 64, "f32"),
    small("f32_d128", 2, 16, 24, 128, "f32"),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_parity(cfg):
    say(f"backward parity {cfg.name}: {cfg.B}x{cfg.heads} L{cfg.L} nb{cfg.nb} d{cfg.d} {cfg.dtype}")
    q, k, v = make_qkv(cfg)
    G, nb, L, d = cfg.BH, cfg.nb, cfg.L, cfg.d
    rng = np.random.default_rng(cfg.index * 31 + d)
    m = random_lists(G, nb, rng)
    cnt, idx = O.kv_lists(m)
    tdt = q.dtype
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(17)).to(tdt)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    o, lse, dq, dk, dv = run_fwd_bwd(qd, kd, vd, dod, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    qn, kn, vn, don = (to_np(t).reshape(G, L, d) for t in (q, k, v, dout))
    # forward log-sum-exp
    ref_lse = O.masked_attention_lse(qn, kn, m, cfg.N)
    gl = to_np(lse).reshape(G, L)
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), live)
    assert np.all(gl[~live] == -np.inf)
    err_lse = float(np.max(np.abs(gl[live] - ref_lse[live])))
    say(f"  lse max-abs {err_lse:.3e}")
    assert err_lse <= TOL_LSE[cfg.dtype]
    # gradients
    rq, rk, rv = O.masked_attention_backward(qn, kn, vn, don, m, cfg.N)
    errs = {n: grad_err(to_np(g).reshape(G, L, d), r) for n, g, r in
            (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))}
    say("  " + "  ".join(f"{n} {e:.3e}" for n, e in errs.items()) + f"  (tol {TOL_GRAD[cfg.dtype]})")
    for n, e in errs.items():
        assert e <= TOL_GRAD[cfg.dtype], n
    # structure: rows of the empty query block and the unkept KV block are exactly zero
    assert np.all(to_np(dq).reshape(G, L, d)[:, 64:128] == 0)
    assert np.all(to_np(dk).reshape(G, L, d)[:, 192:256] == 0)
    assert np.all(to_np(dv).reshape(G, L, d)[:, 192:256] == 0)


def test_backward_on_nabla_mask():
    """The gradient under the lists the mask step itself writes (real content-adaptive
    mask), including the transposed lists built from them."""
    cfg = small("bf16_mask", 4, 24, 32, 128, "bf16", heads=2)
    q, k, v = make_qkv(cfg)
    G, nb, L, d = cfg.BH, cfg.nb, cfg.L, cfg.d
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qf, kf, vf = (nab.reorder(t, cfg.T, cfg.H, cfg.W, cfg.P) for t in (qd, kd, vd))
    cnt, idx = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, cfg.thr)
    dout = torch.randn(qf.shape, generator=torch.Generator().manual_seed(3)).to(qf.dtype).cuda()
    o, lse, dq, dk, dv = run_fwd_bwd(qf, kf, vf, dout, cnt, idx)
    m = lists_to_mask(cnt.cpu().numpy().reshape(G, nb), idx.cpu().numpy().reshape(G, nb, nb))
    say(f"backward on the NABLA mask: kept {m.mean():.3f}")
    args = [to_np(t).reshape(G, L, d) for t in (qf, kf, vf, dout)]
    rq, rk, rv = O.masked_attention_backward(*args, m, cfg.N)
    for n, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = grad_err(to_np(g).reshape(G, L, d), r)
        say(f"  {n} {e:.3e}")
        assert e <= TOL_GRAD["bf16"], n


def test_backward_determinism():
    cfg = CASES[0]
    q, k, v = make_qkv(cfg)
    m = random_lists(cfg.BH, cfg.nb, np.random.default_rng(1))
    cnt, idx = (torch.from_numpy(a).cuda() for a in O.kv_lists(m))
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(2)).to(q.dtype).cuda()
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    a = run_fwd_bwd(qd, kd, vd, dout, cnt, idx)
    b = run_fwd_bwd(qd, kd, vd, dout, cnt, idx)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size():
    """The Wan-1.3B-like layer at full size (the configuration the bench times): dQ of
    sampled query blocks and dK, dV of sampled KV blocks against the oracle, and the
    closed-form sums over every head (dK sums to zero over the keys, dV to the dO of the
    rows that keep something)."""
    cfg = get_config("wan1.3b_480p")
    say(f"backward full size {cfg.name}: {cfg.BH} heads L{cfg.L} nb{cfg.nb}")
    q, k, v = make_qkv(cfg)
    G, nb, L, d, N = cfg.BH, cfg.nb, cfg.L, cfg.d, cfg.N
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qf, kf, vf = (nab.reorder(t, cfg.T, cfg.H, cfg.W, cfg.P) for t in (qd, kd, vd))
    cnt, idx = nab.build_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, N, cfg.thr)
    dout = torch.randn(qf.shape, generator=torch.Generator().manual_seed(5)).to(qf.dtype).cuda()
    o, lse, dq, dk, dv = run_fwd_bwd(qf, kf, vf, dout, cnt, idx)
    say("  gradients computed")
    m = lists_to_mask(cnt.cpu().numpy().reshape(G, nb), idx.cpu().numpy().reshape(G, nb, nb))
    # closed-form sums, every head
    dkn = dk.float().reshape(G, L, d)
    dvn = dv.float().reshape(G, L, d)
    don = dout.float().reshape(G, L, d)
    live = torch.from_numpy(np.repeat(m.any(axis=2), N, axis=1)).cuda()
    sum_dk = dkn.sum(dim=1).abs().max().item()
    sum_dv = (dvn.sum(dim=1) - (don * live[..., None]).sum(dim=1)).abs().max().item()
    scale_k = dkn.abs().max().item()
    say(f"  |sum dK| {sum_dk:.3e} (max |dK| {scale_k:.3e}), |sum dV - sum dO| {sum_dv:.3e}")
    # each is a sum of L bf16-rounded values: allow L * half an ulp of the largest
    assert sum_dk <= L * 2.0 ** -9 * max(1.0, scale_k)
    assert sum_dv <= L * 2.0 ** -9 * max(1.0, dvn.abs().max().item())
    # sampled rows against the oracle, two heads
    rng = np.random.default_rng(13)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for g in (0, G - 1):
        qn, kn, vn, dn = (to_np(t.reshape(G, L, d)[g]) for t in (qf, kf, vf, dout))
        qb_s = sorted({0, nb - 1, *rng.integers(nb, size=3).tolist()})
        kb_s = [int(rng.integers(nb))]
        # the KV blocks' gradients need every query block that keeps them: take those
        # query blocks' full rows of the mask, and the sampled query blocks
        rows = sorted(set(qb_s) | set(np.nonzero(m[g][:, kb_s].any(axis=1))[0].tolist()))
        sub = np.zeros_like(m[g])
        sub[rows] = m[g][rows]
        # dO is zero outside the chosen rows, so the oracle's sums cover exactly them;
        # the GPU's dQ of a chosen row and dK, dV of a chosen KV block only depend on
        # rows that are chosen (for dK, dV) or on the row itself (for dQ)
        dmask = np.zeros((L, 1))
        for i in rows:
            dmask[i * N:(i + 1) * N] = 1.0
        rq, rk, rv = O.masked_attention_backward(qn[None], kn[None], vn[None], (dn * dmask)[None],
                                                 sub[None], N)
        gq = to_np(dq.reshape(G, L, d)[g])
        gk = to_np(dk.reshape(G, L, d)[g])
        gv = to_np(dv.reshape(G, L, d)[g])
        for i in qb_s:
            sl = slice(i * N, (i + 1) * N)
            worst["dq"] = max(worst["dq"], grad_err(gq[sl], rq[0, sl]))
        for j in kb_s:
            sl = slice(j * N, (j + 1) * N)
            worst["dk"] = max(worst["dk"], grad_err(gk[sl], rk[0, sl]))
            worst["dv"] = max(worst["dv"], grad_err(gv[sl], rv[0, sl]))
    say("  sampled: " + "  ".join(f"{n} {e:.3e}" for n, e in worst.items()))
    for n, e in worst.items():
        assert e <= TOL_GRAD["bf16"], n


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["hunyuan_720p_sta", "wan14b_720p_cfg"])
def test_backward_full_size_720p(name):
    """The 720p workloads at full size through the raster-order entry points (the form
    the bench times): the closed-form sums over every head and dQ of sampled query
    blocks against the oracle; dK and dV of a sampled head's least-kept KV block too
    when at most 48 query blocks keep it (each of them needs its whole row in the
    oracle; on these inputs every KV block is kept by hundreds, so there dK and dV are
    checked by the sums, and against the oracle block by block at the Wan-1.3B size)."""
    cfg = get_config(name)
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    G, nb, L, d = cfg.BH, cfg.nb, cfg.L, cfg.d
    say(f"backward full size {cfg.name}: {G} heads L{L} nb{nb}")
    q, k, v = make_qkv(cfg)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    dout = torch.randn(qd.shape, generator=torch.Generator().manual_seed(7)).to(qd.dtype).cuda()
    cnt, idx = nab.build_mask(qd, kd, T, H, W, P, N, cfg.thr, cfg.sta, raster=True)
    o, lse = nab.attn_fwd_raster(qd, kd, vd, cnt, idx, T, H, W, P, N, with_lse=True)
    dq, dk, dv = nab.attn_bwd(qd, kd, vd, o, dout, lse, cnt, idx, N, raster=(T, H, W, P))
    torch.cuda.synchronize()
    say("  gradients computed")
    m = lists_to_mask(cnt.cpu().numpy().reshape(G, nb), idx.cpu().numpy().reshape(G, nb, nb))
    # closed-form sums, every head (token order does not matter for them)
    pi = torch.from_numpy(O.fractal_index(T, H, W, P)).long().cuda()
    live_f = torch.from_numpy(np.repeat(m.any(axis=2), N, axis=1)).cuda()   # fractal order
    live = torch.empty_like(live_f)
    live[:, :] = live_f[:, pi]                                                 # raster token l
    dkn, dvn, don = (t.float().reshape(G, L, d) for t in (dk, dv, dout))
    sum_dk = dkn.sum(dim=1).abs().max().item()
    sum_dv = (dvn.sum(dim=1) - (don * live[..., None]).sum(dim=1)).abs().max().item()
    scale_k = dkn.abs().max().item()
    say(f"  |sum dK| {sum_dk:.3e} (max |dK| {scale_k:.3e}), |sum dV - sum dO| {sum_dv:.3e}")
    assert sum_dk <= L * 2.0 ** -9 * max(1.0, scale_k)
    assert sum_dv <= L * 2.0 ** -9 * max(1.0, dvn.abs().max().item())
    rng = np.random.default_rng(17)
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for g in (0, G - 1):
        qn, kn, vn, dn = (O.reorder(to_np(t.reshape(G, L, d)[g]), T, H, W, P) for t in (qd, kd, vd, dout))
        gq, gk, gv = (O.reorder(to_np(t.reshape(G, L, d)[g]), T, H, W, P) for t in (dq, dk, dv))
        qb_s = sorted({0, nb - 1, int(rng.integers(nb))})
        col = m[g].sum(axis=0)
        kb = int(np.argmin(np.where(col > 0, col, nb + 1)))
        # the oracle's cost grows with the rows that keep the block (each needs its whole
        # row): check dK, dV only where few rows keep it
        check_kv = col[kb] <= 48
        rows = sorted(set(qb_s) | (set(np.nonzero(m[g][:, kb])[0].tolist()) if check_kv else set()))
        sub = np.zeros_like(m[g])
        sub[rows] = m[g][rows]
        dmask = np.zeros((L, 1))
        for i in rows:
            dmask[i * N:(i + 1) * N] = 1.0
        say(f"  head {g}: query blocks {qb_s}, KV block {kb} kept by {int(col[kb])} rows"
            + ("" if check_kv else " (too many for the oracle: dK, dV by the sums only)"))
        rq, rk, rv = O.masked_attention_backward(qn[None], kn[None], vn[None], (dn * dmask)[None], sub[None], N)
        for i in qb_s:
            sl = slice(i * N, (i + 1) * N)
            worst["dq"] = max(worst["dq"], grad_err(gq[sl], rq[0, sl]))
        if check_kv:
            sl = slice(kb * N, (kb + 1) * N)
            worst["dk"] = max(worst["dk"], grad_err(gk[sl], rk[0, sl]))
            worst["dv"] = max(worst["dv"], grad_err(gv[sl], rv[0, sl]))
    say("  sampled: " + "  ".join(f"{n} {e:.3e}" for n, e in worst.items()))
    for n, e in worst.items():
        assert e <= TOL_GRAD["bf16"], n
