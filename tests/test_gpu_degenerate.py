"""GPU: the degenerate grids of the method against the oracle - one block per head, one
block per frame, a single frame under the STA window (whose frame radius then reaches
nothing), an odd number of (batch, head) slices (the attention's last pair has one block)
and a threshold that keeps only each row's largest block.  For each: the mask within
the band rule, attention against the oracle with the GPU's own mask, the raster entry
points bit for bit against the explicit path, the start order, and the gradient against
the oracle's."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
from synth import Config, make_qkv
import block_sparse_attention_blockmean_amd as nab
from parity import TOL_BF16, TOL_F32, check_mask, lists_to_mask, max_abs
from test_gpu_parity import check_pair_schedule

pytestmark = pytest.mark.gpu

TOL_GRAD = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def grid(name, T, H, W, d, dtype, thr, sta=None, heads=3, B=1):
    return Config(name, 21, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=8, N=64, thr=thr,
                  sta=sta, scale_logits=(dtype == "bf16"))


CASES = [
    grid("nb1_bf16", 1, 8, 8, 128, "bf16", 0.2),
    grid("nb1_sta_f32", 1, 8, 8, 64, "f32", 0.2, sta=(3, 3, 3)),
    grid("nb2_frames_f32", 2, 8, 8, 64, "f32", 0.3),
    grid("nb3_frames_sta_bf16", 3, 8, 8, 64, "bf16", 0.1, sta=(1, 1, 1), B=1, heads=1),
    grid("one_frame_sta_bf16", 1, 16, 24, 128, "bf16", 0.2, sta=(3, 3, 3)),
    grid("top_block_only_bf16", 2, 16, 16, 64, "bf16", 0.999),
]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_degenerate_grid(cfg):
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    G, nb, L, d = cfg.BH, cfg.nb, cfg.L, cfg.d
    say(f"degenerate {cfg.name}: {cfg.B}x{cfg.heads} {T}x{H}x{W} d{d} {cfg.dtype} thr{cfg.thr} sta{cfg.sta} nb{nb}")
    q, k, v = make_qkv(cfg)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(31)).to(q.dtype)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    # explicit path
    qf, kf, vf, dof = (nab.reorder(t, T, H, W, P) for t in (qd, kd, vd, dod))
    cnt, idx, sched = nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True)
    of, lse_f = nab.attn_fwd(qf, kf, vf, cnt, idx, N, schedule=sched, with_lse=True)
    gq, gk, gv = nab.attn_bwd(qf, kf, vf, of, dof, lse_f, cnt, idx, N)
    # raster entry points
    cnt_r, idx_r, sched_r = nab.build_mask(qd, kd, T, H, W, P, N, cfg.thr, cfg.sta, with_schedule=True,
                                           raster=True)
    o_r, lse_r = nab.attn_fwd_raster(qd, kd, vd, cnt_r, idx_r, T, H, W, P, N, schedule=sched_r, with_lse=True)
    g_r = nab.attn_bwd(qd, kd, vd, o_r, dod, lse_r, cnt_r, idx_r, N, raster=(T, H, W, P))
    torch.cuda.synchronize()

    # mask against the oracle
    to_np = lambda t: t.detach().float().cpu().numpy()
    qn, kn, vn, don = (O.reorder(to_np(t).reshape(G, L, d), T, H, W, P) for t in (q, k, v, dout))
    ref = O.block_mask(qn, kn, T, H, W, P, N, cfg.thr, cfg.sta)
    cn = cnt.cpu().numpy().reshape(G, nb)
    gmask = lists_to_mask(cn, idx.cpu().numpy().reshape(G, nb, nb))
    mism, band = check_mask(gmask, ref["mask"], ref["A"], cfg.thr)
    assert np.all(cn >= 1), "the largest block of every row is kept"
    if cfg.thr > 0.99:
        assert np.all(cn == 1), "only the largest block clears a threshold this close to 1"
    check_pair_schedule(cfg, sched.cpu().numpy(), cnt.cpu().numpy().reshape(-1))

    # attention and gradient against the oracle, with the GPU's own mask
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    out = O.masked_attention(qn, kn, vn, gmask, N)
    err = max_abs(to_np(of).reshape(G, L, d), out)
    grads = O.masked_attention_backward(qn, kn, vn, don, gmask, N)
    gerr = {n: max_abs(to_np(g).reshape(G, L, d), r) / max(1.0, float(np.max(np.abs(r))))
            for n, g, r in zip(("dq", "dk", "dv"), (gq, gk, gv), grads)}
    say(f"  kept {gmask.mean():.3f}  mismatches {mism}  band {band}  attention {err:.2e}  "
        + "  ".join(f"{n} {e:.2e}" for n, e in gerr.items()))
    assert err <= tol
    for n, e in gerr.items():
        assert e <= TOL_GRAD[cfg.dtype], n

    # the raster entry points give the explicit path's lists, order, output and gradients
    assert torch.equal(cnt_r, cnt) and torch.equal(sched_r, sched)
    for r in range(G * nb):
        c = int(cn.reshape(-1)[r])
        assert torch.equal(idx_r.reshape(-1, nb)[r, :c], idx.reshape(-1, nb)[r, :c])
    back = [nab.reorder(t, T, H, W, P, inverse=True) for t in (of, gq, gk, gv)]
    for name, a, b in zip(("o", "dq", "dk", "dv"), (o_r,) + tuple(g_r), back):
        assert torch.equal(bits(a), bits(b)), name
    pi = torch.from_numpy(O.fractal_index(T, H, W, P)).long().cuda()
    assert torch.equal(bits(lse_r), bits(lse_f[..., pi].contiguous()))
