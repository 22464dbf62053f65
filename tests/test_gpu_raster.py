"""GPU: the raster-order entry points (fractal flattening folded into the addressing)
against the explicit path (nabla_reorder, mask, attention, inverse reorder), bit for bit,
and against the oracle's raster-order whole path."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, T, H, W, d, dtype, thr, sta=None, heads=2, B=1):
    return Config(name, 8, B=B, heads=heads, d=d, dtype=dtype, T=T, H=H, W=W, P=8, N=64, thr=thr,
                  sta=sta, scale_logits=(dtype == "bf16"))


CASES = [
    small("bf16_d128_sta", 5, 24, 40, 128, "bf16", 0.2, sta=(3, 3, 3)),
    small("bf16_d64", 3, 32, 16, 64, "bf16", 0.1, heads=3),
    small("f32_d64", 4, 16, 32, 64, "f32", 0.3),
    small("f32_d128_b2", 2, 16, 16, 128, "f32", 0.05, B=2, heads=1),
]


def both_paths(cfg, q, k, v):
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    qf, kf, vf = (nab.reorder(t, T, H, W, P) for t in (qd, kd, vd))
    ref = nab.build_mask(qf, kf, T, H, W, P, N, cfg.thr, cfg.sta, with_bitmap=True, with_schedule=True)
    of = nab.attn_fwd(qf, kf, vf, ref[0], ref[1], N, schedule=ref[3])
    o_ref = nab.reorder(of, T, H, W, P, inverse=True)
    ras = nab.build_mask(qd, kd, T, H, W, P, N, cfg.thr, cfg.sta, with_bitmap=True, with_schedule=True,
                         raster=True)
    o_ras = nab.attn_fwd_raster(qd, kd, vd, ras[0], ras[1], T, H, W, P, N, schedule=ras[3])
    torch.cuda.synchronize()
    return ref, o_ref, ras, o_ras


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_raster_equals_explicit_reorder(cfg):
    say(f"raster path {cfg.name}: {cfg.B}x{cfg.heads} {cfg.T}x{cfg.H}x{cfg.W} d{cfg.d} {cfg.dtype} sta{cfg.sta}")
    q, k, v = make_qkv(cfg)
    ref, o_ref, ras, o_ras = both_paths(cfg, q, k, v)
    for name, a, b in zip(("kv_count", "kv_index", "bitmap", "schedule"), ref, ras):
        if name == "kv_index":
            # only the first count entries of a row are defined
            cnt = ref[0].reshape(-1).cpu().numpy()
            ia = a.reshape(len(cnt), -1).cpu().numpy()
            ib = b.reshape(len(cnt), -1).cpu().numpy()
            for r in range(len(cnt)):
                assert np.array_equal(ia[r, :cnt[r]], ib[r, :cnt[r]]), r
        else:
            assert torch.equal(a, b), name
    assert torch.equal(bits(o_ref.cpu()), bits(o_ras.cpu()))
    # and the oracle's whole path in raster order, with the GPU's own mask
    G = cfg.BH
    qn, kn, vn = (t.float().numpy().reshape(G, cfg.L, cfg.d) for t in (q, k, v))
    m = lists_to_mask(ras[0].cpu().numpy().reshape(G, cfg.nb), ras[1].cpu().numpy().reshape(G, cfg.nb, cfg.nb))
    qf, kf, vf = (O.reorder(a, cfg.T, cfg.H, cfg.W, cfg.P) for a in (qn, kn, vn))
    out = O.reorder(O.masked_attention(qf, kf, vf, m, cfg.N), cfg.T, cfg.H, cfg.W, cfg.P, inverse=True)
    err = max_abs(o_ras.float().cpu().numpy().reshape(G, cfg.L, cfg.d), out)
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    say(f"  bit-identical to the explicit path; oracle max-abs {err:.3e} (tol {tol})")
    assert err <= tol


def test_raster_full_size_bitwise():
    """The Wan-1.3B-like layer at full size: the raster path gives the explicit path's
    lists and output bit for bit."""
    cfg = get_config("wan1.3b_480p")
    say(f"raster path full size {cfg.name}")
    q, k, v = make_qkv(cfg)
    ref, o_ref, ras, o_ras = both_paths(cfg, q, k, v)
    assert torch.equal(ref[0], ras[0])
    assert torch.equal(ref[2], ras[2])
    assert torch.equal(ref[3], ras[3])
    assert torch.equal(bits(o_ref), bits(o_ras))


def grad_err(gpu, ref):
    return max_abs(gpu, ref) / max(1.0, float(np.max(np.abs(ref))))


def backward_paths(cfg, q, k, v, dout):
    """Forward with log-sum-exp and gradient of raster-ordered tensors through the raster
    entry points, and through reorder + the fractal entry points + inverse reorder, under
    the raster mask step's lists."""
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.P, cfg.N
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    cnt, idx = nab.build_mask(qd, kd, T, H, W, P, N, cfg.thr, cfg.sta, raster=True)
    o_r, lse_r = nab.attn_fwd_raster(qd, kd, vd, cnt, idx, T, H, W, P, N, with_lse=True)
    g_r = nab.attn_bwd(qd, kd, vd, o_r, dod, lse_r, cnt, idx, N, raster=(T, H, W, P))
    qf, kf, vf, dof = (nab.reorder(t, T, H, W, P) for t in (qd, kd, vd, dod))
    o_f, lse_f = nab.attn_fwd(qf, kf, vf, cnt, idx, N, with_lse=True)
    g_f = nab.attn_bwd(qf, kf, vf, o_f, dof, lse_f, cnt, idx, N)
    back = [nab.reorder(t, T, H, W, P, inverse=True) for t in (o_f,) + tuple(g_f)]
    pi = torch.from_numpy(O.fractal_index(T, H, W, P)).long().cuda()
    lse_back = lse_f[..., pi]       # raster token l sits at fractal position pi[l]
    torch.cuda.synchronize()
    return (cnt, idx), (o_r, lse_r) + tuple(g_r), (back[0], lse_back) + tuple(back[1:])


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_raster_backward_equals_explicit_reorder(cfg):
    """The raster forward-with-lse and gradient give the explicit path's O, lse, dQ, dK,
    dV bit for bit, and match the oracle's gradient in raster order."""
    say(f"raster backward {cfg.name}: {cfg.B}x{cfg.heads} {cfg.T}x{cfg.H}x{cfg.W} d{cfg.d} {cfg.dtype}")
    q, k, v = make_qkv(cfg)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(23)).to(q.dtype)
    (cnt, idx), ras, ref = backward_paths(cfg, q, k, v, dout)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ras, ref):
        assert torch.equal(bits(a.cpu()), bits(b.cpu())), name
    G, L, d = cfg.BH, cfg.L, cfg.d
    m = lists_to_mask(cnt.cpu().numpy().reshape(G, cfg.nb), idx.cpu().numpy().reshape(G, cfg.nb, cfg.nb))
    args = [O.reorder(t.float().numpy().reshape(G, L, d), cfg.T, cfg.H, cfg.W, cfg.P) for t in (q, k, v, dout)]
    grads = O.masked_attention_backward(*args, m, cfg.N)
    tol = {"bf16": 2e-2, "f32": 1e-4}[cfg.dtype]
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), ras[2:], grads):
        r_ras = O.reorder(r, cfg.T, cfg.H, cfg.W, cfg.P, inverse=True)
        errs[name] = grad_err(g.float().cpu().numpy().reshape(G, L, d), r_ras)
    say("  bit-identical to the explicit path; oracle " + "  ".join(f"{n} {e:.3e}" for n, e in errs.items())
        + f" (tol {tol})")
    for name, e in errs.items():
        assert e <= tol, name


def test_raster_backward_full_size_bitwise():
    """The Wan-1.3B-like layer at full size: the raster gradient equals the explicit
    path's bit for bit."""
    cfg = get_config("wan1.3b_480p")
    say(f"raster backward full size {cfg.name}")
    q, k, v = make_qkv(cfg)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(29)).to(q.dtype)
    _, ras, ref = backward_paths(cfg, q, k, v, dout)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ras, ref):
        assert torch.equal(bits(a), bits(b)), name
