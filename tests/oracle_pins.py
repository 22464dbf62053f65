"""Pins of the oracle against facts that the pages and plain mathematics fix.

Each ``pin_*`` raises AssertionError when the oracle disagrees.  They look the
oracle functions up at call time (``O.name``), so the mutation tests can plant a
mistake in the oracle and check that some pin catches it.
"""
from __future__ import annotations

import itertools

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import oracle.nabla_oracle as O
from conftest import read_golden


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- reorder

def pin_reorder_golden():
    lines = read_golden("fractal_T2_H4_W4_P2.txt")
    T, H, W, P = map(int, lines[0].split())
    seq = np.array(list(map(int, lines[1].split())))
    L = T * H * W
    x = np.arange(L, dtype=np.int64)[:, None]
    y = O.reorder(x, T, H, W, P)
    assert np.array_equal(y[:, 0], seq), (y[:, 0], seq)
    assert np.array_equal(O.reorder(y, T, H, W, P, inverse=True)[:, 0], np.arange(L))


def pin_reorder_roundtrip():
    rng = _rng(1)
    for T, H, W, P in [(1, 8, 8, 2), (3, 8, 16, 4), (2, 16, 8, 8), (2, 6, 9, 3), (1, 4, 4, 1)]:
        L = T * H * W
        x = rng.standard_normal((2, L, 3)).astype(np.float32)
        y = O.reorder(x, T, H, W, P)
        z = O.reorder(y, T, H, W, P, inverse=True)
        assert np.array_equal(z, x)
        pi = O.fractal_index(T, H, W, P)
        assert np.array_equal(np.sort(pi), np.arange(L)), "not a bijection"


def pin_reorder_identity_cases():
    x = np.arange(2 * 8 * 8, dtype=np.int64)[:, None]
    assert np.array_equal(O.reorder(x, 2, 8, 8, 1), x), "P = 1 must keep raster order"
    assert np.array_equal(O.reorder(x, 2, 8, 8, 8), x), "P = H = W must keep raster order"


def pin_reorder_runs_are_patches():
    T, H, W, P = 3, 8, 12, 4
    L = T * H * W
    y = O.reorder(np.arange(L, dtype=np.int64)[:, None], T, H, W, P)[:, 0]
    t, rem = np.divmod(y, H * W)
    yy, xx = np.divmod(rem, W)
    prev_t = -1
    for r in range(L // (P * P)):
        sl = slice(r * P * P, (r + 1) * P * P)
        coords = set(zip(t[sl], yy[sl] // P, xx[sl] // P))
        assert len(coords) == 1, "a run of P*P tokens must be one patch of one frame"
        tt = int(t[sl][0])
        assert tt >= prev_t, "time order must be kept"
        prev_t = tt


# ---------------------------------------------------------------- pooling / map

def pin_pool_tile_mean():
    """Pooled logit (i, j) = mean of the dense logits over the N x N tile (bilinearity)."""
    rng = _rng(2)
    for L, N, d in [(256, 64, 16), (192, 64, 8), (48, 16, 4)]:
        q = rng.standard_normal((L, d)).astype(np.float32) + 0.3
        k = rng.standard_normal((L, d)).astype(np.float32) * 1.7 - 0.2
        scale = 1.0 / np.sqrt(d)
        S = O.pooled_logits(O.block_mean(q, N), O.block_mean(k, N), scale)
        nb = L // N
        dense = np.zeros((L, L))
        for a in range(L):
            for b in range(L):
                dense[a, b] = scale * sum(float(q[a, c]) * float(k[b, c]) for c in range(d))
        tile_mean = dense.reshape(nb, N, nb, N).mean(axis=(1, 3))
        assert np.allclose(S, tile_mean, rtol=1e-5, atol=1e-6), np.max(np.abs(S - tile_mean))


def pin_pool_constant():
    # a dyadic constant sums exactly, so the mean is exact
    x = np.full((2, 256, 8), 0.75, dtype=np.float32)
    p = O.block_mean(x, 64)
    assert p.shape == (2, 4, 8)
    assert np.all(p == np.float32(0.75)), p
    # otherwise within the textbook bound of a sequential float32 sum, (N-1) u |c|
    x = np.full((1, 128, 4), 0.7, dtype=np.float32)
    p = O.block_mean(x, 64)
    assert np.all(np.abs(p.astype(np.float64) - 0.7) <= 63 * 2.0 ** -24 * 0.7 + 2.0 ** -24), p


def pin_softmax():
    rng = _rng(3)
    S = (rng.standard_normal((5, 37)) * 4).astype(np.float32)
    A = O.row_softmax(S)
    assert np.all(np.abs(A.sum(-1) - 1.0) <= 37 * 2.0 ** -24 + 1e-7)
    ref = scipy.special.softmax(S.astype(np.float64), axis=-1)
    assert np.max(np.abs(A - ref)) <= 1e-6
    A2 = O.row_softmax(S + np.float32(3.5))
    assert np.max(np.abs(A2 - A)) <= 1e-6
    assert np.all(np.argmax(A, -1) == np.argmax(S, -1))


# ---------------------------------------------------------------- CDF threshold

def _golden_cdf_rows():
    rows = []
    for ln in read_golden("cdf_rows.txt"):
        thr, vals, bits, fs = [s.strip() for s in ln.split("|")]
        rows.append((float(thr), np.array(vals.split(), dtype=np.float32),
                     np.array(bits.split(), dtype=int).astype(bool),
                     np.array(fs.split(), dtype=np.float32)))
    return rows


def pin_cdf_golden():
    for thr, row, bits, fs in _golden_cdf_rows():
        Fv = O.cdf_values(row[None, :])[0]
        assert np.array_equal(Fv, fs), (row, Fv, fs)
        keep = O.cdf_keep(row[None, :], thr)[0]
        assert np.array_equal(keep, bits), (thr, row, keep, bits)


def _brute_F(A):
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[-1]
    out = np.zeros_like(A)
    for r in range(A.shape[0]):
        for j in range(n):
            out[r, j] = sum(A[r, k] for k in range(n) if A[r, k] <= A[r, j])
    return out


def pin_cdf_bruteforce():
    rng = _rng(4)
    A = rng.random((40, 12))
    A[:, 3] = A[:, 7]            # forced ties
    A[::3, 1] = A[::3, 2] = A[::3, 5]
    A /= A.sum(-1, keepdims=True)
    assert np.max(np.abs(O.cdf_values(A) - _brute_F(A))) <= 1e-12


def pin_cdf_invariants():
    rng = _rng(5)
    S = (rng.standard_normal((60, 24)) * 3).astype(np.float32)
    S[:10, 4] = S[:10, 9]
    A = O.row_softmax(S)
    assert O.cdf_keep(A, 0.0).all(), "thr = 0 keeps every block"
    prev = None
    for thr in [0.0, 0.05, 0.1, 0.2, 0.4, 0.7, 0.95]:
        keep = O.cdf_keep(A, thr)
        kept_mass = np.where(keep, A, 0).astype(np.float64).sum(-1)
        assert np.all(kept_mass >= 1.0 - thr - 1e-5), "kept mass must reach 1 - thr"
        assert np.all(keep[np.arange(len(A)), np.argmax(A, -1)]), "row max is always kept"
        for r in range(len(A)):
            # minimality: re-adding the smallest kept group would be needed, i.e. the
            # dropped mass plus that group exceeds thr
            kept_vals = A[r][keep[r]]
            vmin = kept_vals.min()
            dropped_plus = A[r][A[r] <= vmin].astype(np.float64).sum()
            assert dropped_plus > thr - 1e-6
        if prev is not None:
            assert np.all(prev >= keep), "kept set shrinks as thr grows"
        prev = keep
    uni = np.full((1, 16), 1.0 / 16, dtype=np.float32)
    assert O.cdf_keep(uni, 0.9).all(), "a uniform row keeps every block"


# ---------------------------------------------------------------- STA

def pin_sta_counts():
    for ln in read_golden("sta_counts.txt"):
        T, H, W, P, wt, wh, ww, n = map(int, ln.split())
        M = O.sta_mask(T, H, W, P, P * P, (wt, wh, ww))
        assert int(M.sum()) == n, (ln, int(M.sum()))
        assert np.array_equal(M, M.T)
        assert M.diagonal().all()


def pin_sta_brute():
    """Against the tile numbering that the fractal order implies (block i sits at
    tile (t, h, w) with i = (t*nH + h)*nW + w), enumerated directly."""
    T, H, W, P = 3, 16, 24, 8
    nH, nW = H // P, W // P
    M = O.sta_mask(T, H, W, P, P * P, (3, 1, 3))
    nb = T * nH * nW
    ref = np.zeros((nb, nb), dtype=bool)
    for (t1, h1, w1), (t2, h2, w2) in itertools.product(
            itertools.product(range(T), range(nH), range(nW)), repeat=2):
        i = (t1 * nH + h1) * nW + w1
        j = (t2 * nH + h2) * nW + w2
        ref[i, j] = abs(t1 - t2) <= 1 and h1 == h2 and abs(w1 - w2) <= 1
    assert np.array_equal(M, ref)


def pin_sta_union():
    """M = M_nabla OR M_STA: the mask with a window is the CDF mask with every block of
    the window added, so it contains each part, and on a grid where each part holds
    blocks the other lacks it is strictly larger than both.  The window part is
    enumerated here from tile coordinates (block i = (t*nH + h)*nW + w, its 1 x P x P
    tile), independently of sta_mask."""
    rng = _rng(12)
    T, H, W, P, N, d = 3, 16, 24, 8, 64, 16
    nH, nW = H // P, W // P
    L = T * H * W
    base = rng.standard_normal((1, L, d)).astype(np.float32)
    q = (base + 0.3 * rng.standard_normal((1, L, d))).astype(np.float32)
    k = (base + 0.3 * rng.standard_normal((1, L, d))).astype(np.float32)
    win = (1, 3, 1)
    plain = O.block_mask(q, k, T, H, W, P, N, 0.3)
    both = O.block_mask(q, k, T, H, W, P, N, 0.3, sta=win)
    nb = T * nH * nW
    ref = np.zeros((nb, nb), dtype=bool)
    for (t1, h1, w1), (t2, h2, w2) in itertools.product(
            itertools.product(range(T), range(nH), range(nW)), repeat=2):
        ref[(t1 * nH + h1) * nW + w1, (t2 * nH + h2) * nW + w2] = t1 == t2 and abs(h1 - h2) <= 1 and w1 == w2
    m_cdf = plain["mask"][0]
    assert np.array_equal(both["mask_nabla"][0], m_cdf)
    assert np.array_equal(both["mask"][0], m_cdf | ref)
    assert np.all(both["mask"][0] >= m_cdf) and np.all(both["mask"][0] >= ref)
    assert (ref & ~m_cdf).any() and (m_cdf & ~ref).any(), "each part must add blocks the other lacks"


# ---------------------------------------------------------------- lists

def pin_kv_lists():
    rng = _rng(6)
    m = rng.random((3, 10, 10)) < 0.4
    m[:, np.arange(10), np.arange(10)] = True
    cnt, idx = O.kv_lists(m)
    assert np.array_equal(cnt, m.sum(-1))
    for g in range(3):
        for i in range(10):
            row = idx[g, i, :cnt[g, i]]
            assert np.all(np.diff(row) > 0), "ascending and unique"
            assert np.array_equal(row, np.nonzero(m[g, i])[0])
            assert np.all(idx[g, i, cnt[g, i]:] == -1)
    assert np.array_equal(O.mask_from_lists(cnt, idx), m)


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, tok_mask=None, scale=None):
    qt, kt, vt = (torch.from_numpy(np.asarray(a, dtype=np.float64))[None] for a in (q, k, v))
    am = None if tok_mask is None else torch.from_numpy(tok_mask)[None]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)[0].numpy()


def pin_attention_dense():
    rng = _rng(7)
    G, L, N, d = 2, 256, 64, 16
    q, k, v = (rng.standard_normal((G, L, d)).astype(np.float32) for _ in range(3))
    full = np.ones((G, L // N, L // N), dtype=bool)
    out = O.masked_attention(q, k, v, full, N)
    ref = _sdpa(q, k, v)
    assert np.max(np.abs(out - ref)) <= 1e-12


def pin_attention_masked():
    rng = _rng(8)
    G, L, N, d = 2, 320, 64, 8
    nb = L // N
    q, k, v = (rng.standard_normal((G, L, d)).astype(np.float32) * 2 for _ in range(3))
    m = rng.random((G, nb, nb)) < 0.5
    m[:, np.arange(nb), (np.arange(nb) * 3) % nb] = True
    out = O.masked_attention(q, k, v, m, N, scale=0.3)
    tok = np.stack([np.kron(m[g], np.ones((N, N), dtype=bool)) for g in range(G)])
    ref = _sdpa(q, k, v, tok, scale=0.3)
    assert np.max(np.abs(out - ref)) <= 1e-12
    # convex hull: every output channel lies between the min and max of the kept values
    for g in range(G):
        for i in range(nb):
            toks = np.concatenate([np.arange(j * N, (j + 1) * N) for j in np.nonzero(m[g, i])[0]])
            lo, hi = v[g, toks].min(0), v[g, toks].max(0)
            o = out[g, i * N:(i + 1) * N]
            assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def pin_attention_diagonal():
    rng = _rng(9)
    L, N, d = 256, 64, 8
    q, k, v = (rng.standard_normal((1, L, d)).astype(np.float32) for _ in range(3))
    m = np.eye(L // N, dtype=bool)[None]
    out = O.masked_attention(q, k, v, m, N)
    for i in range(L // N):
        sl = slice(i * N, (i + 1) * N)
        ref = _sdpa(q[0, sl], k[0, sl], v[0, sl])
        assert np.max(np.abs(out[0, sl] - ref)) <= 1e-12


def pin_forward_thr0_is_full_attention():
    """thr = 0 keeps every block; reorder -> attention -> inverse reorder is then
    plain full attention in raster order."""
    rng = _rng(10)
    T, H, W, P, N, d = 2, 16, 16, 8, 64, 16
    L = T * H * W
    q, k, v = (rng.standard_normal((2, L, d)).astype(np.float32) for _ in range(3))
    res = O.forward(q, k, v, T, H, W, P, N, thr=0.0)
    assert res["mask"].all()
    ref = _sdpa(q, k, v)
    assert np.max(np.abs(res["out"] - ref)) <= 1e-12


def pin_forward_permutation_equivariance():
    """Attention in fractal order, mapped back, equals raster attention under the
    token mask carried back through the same permutation."""
    rng = _rng(11)
    T, H, W, P, N, d = 2, 16, 16, 8, 64, 8
    L = T * H * W
    q, k, v = (rng.standard_normal((1, L, d)).astype(np.float32) for _ in range(3))
    res = O.forward(q, k, v, T, H, W, P, N, thr=0.3)
    assert not res["mask"].all()
    pi = O.fractal_index(T, H, W, P)
    blk = pi // N                                  # block of each raster token
    tok = res["mask"][0][blk[:, None], blk[None, :]]
    ref = _sdpa(q, k, v, tok[None])
    assert np.max(np.abs(res["out"] - ref)) <= 1e-12


def pin_mask_precision_band():
    """The float32 mask equals the float64 one except where F lies within 1e-4 of thr."""
    from synth import get_config, make_head
    cfg = get_config("tiny")
    q, k, _ = make_head(cfg, 0, 0)
    qf = O.reorder(q, cfg.T, cfg.H, cfg.W, cfg.P)
    kf = O.reorder(k, cfg.T, cfg.H, cfg.W, cfg.P)
    for thr in (0.05, 0.1, 0.2, 0.5):
        m32 = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, dtype=np.float32)
        m64 = O.block_mask(qf, kf, cfg.T, cfg.H, cfg.W, cfg.P, cfg.N, thr, dtype=np.float64)
        diff = m32["mask"] != m64["mask"]
        assert np.all(np.abs(m64["F"][diff] - thr) <= 1e-4)
        assert np.max(np.abs(m32["F"] - m64["F"])) <= 1e-5


# ---------------------------------------------------------------- backward (gradient of attention)

def _tok_mask(m, N):
    return np.stack([np.kron(m[g], np.ones((N, N), dtype=bool)) for g in range(m.shape[0])])


def _autograd_grads(q, k, v, dout, tok, scale):
    """Gradients of sum(O * dout) by torch autograd through the float64 SDPA math
    path with a boolean token mask (an implementation independent of the oracle)."""
    qt, kt, vt = (torch.from_numpy(np.asarray(a, dtype=np.float64)).requires_grad_(True)
                  for a in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(tok), scale=scale)
    (o * torch.from_numpy(np.asarray(dout, dtype=np.float64))).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_lse_logsumexp():
    rng = _rng(20)
    G, L, N, d = 2, 320, 64, 8
    nb = L // N
    q, k = (rng.standard_normal((G, L, d)).astype(np.float32) * 2 for _ in range(2))
    m = rng.random((G, nb, nb)) < 0.4
    m[:, np.arange(nb), np.arange(nb)] = True
    m[1, 2] = False                                   # an empty row
    lse = O.masked_attention_lse(q, k, m, N, scale=0.4)
    tok = _tok_mask(m, N)
    s = np.einsum("gad,gbd->gab", q.astype(np.float64), k.astype(np.float64)) * 0.4
    ref = scipy.special.logsumexp(np.where(tok, s, -np.inf), axis=-1)
    ok = np.isfinite(ref)
    assert np.array_equal(ok, np.isfinite(lse))
    assert np.all(lse[~ok] == -np.inf)
    assert np.max(np.abs(lse[ok] - ref[ok])) <= 1e-12


def pin_backward_autograd():
    rng = _rng(21)
    G, L, N, d = 2, 320, 64, 8
    nb = L // N
    q, k, v, do = (rng.standard_normal((G, L, d)).astype(np.float32) * 1.5 for _ in range(4))
    for trial, density in enumerate((1.0, 0.45)):
        m = rng.random((G, nb, nb)) < density
        m[:, np.arange(nb), (np.arange(nb) * 2 + trial) % nb] = True   # no empty row
        dq, dk, dv = O.masked_attention_backward(q, k, v, do, m, N, scale=0.35)
        rq, rk, rv = _autograd_grads(q, k, v, do, _tok_mask(m, N), 0.35)
        for a, b in ((dq, rq), (dk, rk), (dv, rv)):
            assert np.max(np.abs(a - b)) <= 1e-10 * max(1.0, np.max(np.abs(b)))


def pin_backward_finite_difference():
    rng = _rng(22)
    G, L, N, d = 1, 192, 64, 4
    nb = L // N
    q, k, v, do = (rng.standard_normal((G, L, d)) for _ in range(4))
    m = np.array([[[1, 0, 1], [1, 1, 0], [0, 0, 1]]], dtype=bool)
    scale = 0.7
    dq, dk, dv = O.masked_attention_backward(q, k, v, do, m, N, scale=scale)

    def f(q_, k_, v_):
        return float(np.sum(O.masked_attention(q_, k_, v_, m, N, scale=scale) * do))

    eps = 1e-6
    for which, g in ((0, dq), (1, dk), (2, dv)):
        for _ in range(3):
            u = rng.standard_normal((G, L, d))
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + eps * u
            args_m[which] = args_m[which] - eps * u
            fd = (f(*args_p) - f(*args_m)) / (2 * eps)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def pin_backward_sums_and_empty_rows():
    """Rows of dS sum to zero, so the dK of a head sums to zero over its keys; P's
    rows sum to one, so dV sums to the dO of the rows that keep something.  A query
    block with no kept block passes no gradient at all."""
    rng = _rng(23)
    G, L, N, d = 2, 384, 64, 8
    nb = L // N
    q, k, v, do = (rng.standard_normal((G, L, d)) for _ in range(4))
    m = rng.random((G, nb, nb)) < 0.5
    m[:, np.arange(nb), np.arange(nb)] = True
    m[0, 3] = False
    dq, dk, dv = O.masked_attention_backward(q, k, v, do, m, N)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-10
    live = np.repeat(m.any(axis=2), N, axis=1)          # [G, L] rows that keep a block
    assert np.max(np.abs(dv.sum(axis=1) - (do * live[..., None]).sum(axis=1))) <= 1e-10
    assert np.all(dq[0, 3 * N:4 * N] == 0)
    m2 = m.copy()
    m2[0, 3] = False
    do2 = do.copy()
    do2[0, 3 * N:4 * N] = rng.standard_normal((N, d))   # dO of the empty block is irrelevant
    dq2, dk2, dv2 = O.masked_attention_backward(q, k, v, do2, m2, N)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


# ---------------------------------------------------------------- SIP (sampling + HT weights)

def _sip_rows(rng):
    rows = [rng.random(24) ** 4, rng.random(40), np.full(16, 1.0 / 16), rng.random(30) ** 8]
    z = rng.random(20)
    z[[3, 7, 11]] = 0.0                                   # zero-score blocks
    rows.append(z)
    t = rng.random(18)
    t[[2, 5, 9]] = t.max()                                # tied maxima: the smallest index is certain
    rows.append(t)
    return [r / r.sum() for r in rows]


def pin_sip_probabilities():
    """Budget, caps, the certain top block, monotonicity, and proportionality to the
    score among the blocks that are neither certain nor zero."""
    rng = _rng(30)
    for A in _sip_rows(rng):
        nb = len(A)
        top = int(np.argmax(A))
        pos = int(np.count_nonzero(A))
        for k in (1, 2, 5, nb // 2, nb - 1, nb, nb + 3):
            pi = O.sip_probabilities(A, k)
            assert np.all(pi >= 0) and np.all(pi <= 1 + 1e-15)
            assert pi[top] == 1.0
            if k >= nb:
                assert np.all(pi == 1.0)
                continue
            assert abs(pi.sum() - min(k, pos)) <= 1e-9, (k, pi.sum(), pos)
            others = np.array([j for j in range(nb) if j != top])
            a, p = A[others], pi[others]
            order = np.argsort(a)
            assert np.all(np.diff(p[order]) >= -1e-15), "pi must not decrease with the score"
            mid = (p > 0) & (p < 1)
            if mid.sum() >= 2:
                ratio = p[mid] / a[mid]
                assert np.max(ratio) - np.min(ratio) <= 1e-9 * np.max(ratio)
            assert np.all(p[a == 0] == 0)
            if k > 1 and mid.any():
                assert np.all(p[~mid & (a > 0)] == 1.0)


def pin_sip_horvitz_thompson_unbiased():
    """Kept blocks weighted by exp(logw) = 1/pi give an unbiased sum: the expectation
    over all inclusion outcomes (independent, P(keep j) = pi_j) of sum_j keep_j x_j / pi_j
    equals sum_j x_j, enumerated exactly on small rows."""
    rng = _rng(31)
    for nb, k in ((6, 3), (7, 2), (8, 5)):
        A = rng.random(nb) ** 3
        A /= A.sum()
        pi = O.sip_probabilities(A, k)
        x = rng.standard_normal(nb)
        expect = 0.0
        total_p = 0.0
        for outcome in range(1 << nb):
            keep = np.array([(outcome >> j) & 1 for j in range(nb)], dtype=bool)
            prob = np.prod(np.where(keep, pi, 1.0 - pi))
            if prob == 0.0:
                continue
            # uniforms that realise this outcome under the rule keep iff u < pi
            u = np.where(keep, 0.0, np.minimum(pi + (1.0 - pi) * 0.5, np.nextafter(1.0, 0.0)))
            m, logw, _ = O.sip_mask(A[None], k, u[None])
            assert np.array_equal(m[0], keep)
            expect += prob * float(np.sum(m[0] * np.exp(logw[0]) * x))
            total_p += prob
        assert abs(total_p - 1.0) <= 1e-12
        assert abs(expect - x[pi > 0].sum()) <= 1e-10 * max(1.0, np.abs(x).sum())


def pin_weighted_attention_sdpa():
    """Per-tile logit shifts = SDPA with an additive float mask (shift on kept tokens,
    -inf on dropped ones)."""
    rng = _rng(32)
    G, L, N, d = 2, 320, 64, 8
    nb = L // N
    q, k, v = (rng.standard_normal((G, L, d)).astype(np.float32) for _ in range(3))
    m = rng.random((G, nb, nb)) < 0.5
    m[:, np.arange(nb), np.arange(nb)] = True
    logw = np.where(m, rng.random((G, nb, nb)) * 3.0, 0.0)
    out = O.weighted_block_attention(q, k, v, m, logw, N, scale=0.4)
    bias = np.where(m, logw, -np.inf)
    tb = np.stack([np.kron(bias[g], np.ones((N, N))) for g in range(G)])
    qt, kt, vt = (torch.from_numpy(a.astype(np.float64))[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(tb)[None], scale=0.4)[0].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def pin_sip_full_budget_is_plain_attention():
    """With a budget of every block, every block is certain with shift 0: the SIP path
    is the plain block attention over all blocks, i.e. dense attention."""
    rng = _rng(33)
    G, L, N, d = 1, 256, 64, 8
    nb = L // N
    q, k, v = (rng.standard_normal((G, L, d)).astype(np.float32) for _ in range(3))
    A = rng.random((G, nb, nb))
    A /= A.sum(-1, keepdims=True)
    m, logw, pi = O.sip_mask(A, nb, rng.random((G, nb, nb)))
    assert m.all() and np.all(logw == 0) and np.all(pi == 1)
    out = O.weighted_block_attention(q, k, v, m, logw, N)
    assert np.max(np.abs(out - _sdpa(q, k, v))) <= 1e-12


# ---------------------------------------------------------------- IBCS (intra-block clustering)

def pin_ibcs_identical_queries_is_block_mean():
    """A block whose queries are all equal forms one cluster whose centroid is the block
    mean: IBCS's row is then exactly NABLA's pooled softmax row."""
    rng = _rng(40)
    G, L, N, d = 1, 256, 64, 16
    nb = L // N
    q = np.repeat(rng.standard_normal((G, nb, 1, d)), N, axis=2).reshape(G, L, d).astype(np.float32)
    k = rng.standard_normal((G, L, d)).astype(np.float32) * 2
    A = O.ibcs_scores(q, k, N, scale=0.3)
    qp = O.block_mean(q, N, np.float64)
    kp = O.block_mean(k, N, np.float64)
    S = qp @ kp.transpose(0, 2, 1) * 0.3
    ref = np.exp(S - S.max(-1, keepdims=True))
    ref /= ref.sum(-1, keepdims=True)
    assert np.max(np.abs(A - ref)) <= 1e-12
    for i in range(nb):
        cent, w = O.ibcs_clusters(q[0, i * N:(i + 1) * N])
        # every distance ties at 0, so every query joins cluster 0, whose mean is the query
        assert w[0] == 1.0 and np.all(w[1:] == 0.0)
        assert np.array_equal(cent[0], q[0, i * N].astype(np.float64))


def pin_ibcs_separated_groups():
    """Eight well-separated groups of eight consecutive queries (the initial centroids
    fall one per group) are recovered: weights 1/8, centroids the group means."""
    rng = _rng(41)
    N, d = 64, 12
    centers = rng.standard_normal((8, d)) * 20
    x = (np.repeat(centers, 8, axis=0) + rng.standard_normal((N, d)) * 0.1).astype(np.float32)
    perm = np.concatenate([[g * 8] for g in range(8)] + [[g * 8 + r for r in range(1, 8)] for g in range(8)])
    cent, w = O.ibcs_clusters(x)
    assert np.allclose(w, 1.0 / 8)
    assert np.max(np.abs(cent - x.reshape(8, 8, d).mean(axis=1))) <= 1e-5
    assert len(perm) == N


def pin_ibcs_matches_library_kmeans():
    """Lloyd's k-means from the same initial centroids, by scikit-learn's implementation."""
    from sklearn.cluster import KMeans
    rng = _rng(42)
    for trial in range(4):
        N, d = 64, 16
        x = (rng.standard_normal((N, d)) + (rng.random((N, 1)) > 0.5) * 3).astype(np.float32)
        cent, w = O.ibcs_clusters(x)
        init = x[np.arange(8) * 8].astype(np.float64)
        km = KMeans(n_clusters=8, init=init, n_init=1, max_iter=O.IBCS_ITERS, tol=0.0,
                    algorithm="lloyd").fit(x.astype(np.float64))
        assert np.max(np.abs(cent - km.cluster_centers_)) <= 1e-10, trial
        # the weights come from the last assignment, the one made against the centroids of
        # the previous round: scikit-learn's final labels after one round fewer
        km3 = KMeans(n_clusters=8, init=init, n_init=1, max_iter=O.IBCS_ITERS - 1, tol=0.0,
                     algorithm="lloyd").fit(x.astype(np.float64))
        assert np.array_equal(w, np.bincount(km3.labels_, minlength=8) / N), trial


def pin_ibcs_matches_library_kmeans_128():
    """The page's 128-query groups: Lloyd's k-means of 128 queries from rows 0, 16, ...,
    112, against scikit-learn's implementation."""
    from sklearn.cluster import KMeans
    rng = _rng(44)
    for trial in range(3):
        n, d = 128, 12
        x = (rng.standard_normal((n, d)) + (rng.random((n, 1)) > 0.6) * 4).astype(np.float32)
        cent, w = O.ibcs_clusters(x)
        init = x[np.arange(8) * 16].astype(np.float64)
        km = KMeans(n_clusters=8, init=init, n_init=1, max_iter=O.IBCS_ITERS, tol=0.0,
                    algorithm="lloyd").fit(x.astype(np.float64))
        # (scikit-learn's labels_ come from one more assignment against the final
        # centres; the weights here are those of the assignment that made them, which
        # the closed-form pin below checks)
        assert np.max(np.abs(cent - km.cluster_centers_)) <= 1e-10, trial


def pin_ibcs_group128_scores_closed_form():
    """qn = 128: each group of two 64-token blocks holds 8 well-separated centres, 16
    consecutive queries each (the initial rows 0, 16, ... fall one per centre), so the
    clusters are the centres with weight 1/8 and both blocks of the group score
    A_j = 1/8 sum_c softmax_j(scale c . Kp_j), computed here from the centres alone.
    Clustering each 64-block on its own (4 centres, 2 initial rows each) gives other
    rows."""
    rng = _rng(45)
    G, T, N, d, scale = 1, 4, 64, 8, 0.2
    L = T * N * 2
    nb = L // N
    centers = rng.standard_normal((L // 128, 8, d)) * 10
    q = np.repeat(centers, 16, axis=1).reshape(1, L, d)
    q = (q + rng.standard_normal(q.shape) * 1e-3).astype(np.float32)
    k = rng.standard_normal((G, L, d)).astype(np.float32)
    A = O.ibcs_scores(q, k, N, scale, qn=128)
    kp = k.astype(np.float64).reshape(nb, N, d).mean(axis=1)
    for gi in range(L // 128):
        mu = q[0, gi * 128:(gi + 1) * 128].astype(np.float64).reshape(8, 16, d).mean(axis=1)
        S = mu @ kp.T * scale
        P = np.exp(S - S.max(-1, keepdims=True))
        P /= P.sum(-1, keepdims=True)
        ref = P.mean(axis=0)
        for b in (2 * gi, 2 * gi + 1):
            assert np.max(np.abs(A[0, b] - ref)) <= 1e-5, (gi, b)
    A64 = O.ibcs_scores(q, k, N, scale)
    assert np.max(np.abs(A64 - A)) > 1e-3


def pin_ibcs_margin_closed_form():
    """The clustering margin of a group (second-smallest minus smallest squared distance,
    over the second-smallest, minimised over queries and rounds) in closed form: eight
    distinct queries that are themselves the eight initial centroids each sit at distance
    0 from their own centroid, so every margin is exactly 1 and each cluster keeps one
    query; a query repeated at rows 0 and 1 ties at distance 0 between clusters 0 and 1,
    so the margin is 0, both copies join cluster 0 (lowest index on ties) and cluster 1
    stays empty."""
    rng = _rng(47)
    x = rng.standard_normal((8, 5)) * 3
    cent, w, gap = O.ibcs_clusters(x, return_gap=True)
    assert gap == 1.0 and np.all(w == 1.0 / 8)
    assert np.array_equal(cent, x)
    y = x.copy()
    y[1] = y[0]
    cent, w, gap = O.ibcs_clusters(y, return_gap=True)
    assert gap == 0.0
    assert w[0] == 2.0 / 8 and w[1] == 0.0 and np.all(w[2:] == 1.0 / 8)
    # batched form, per group, and per row of ibcs_scores (both query blocks of a group)
    cents, ws, gaps = O.ibcs_clusters(np.stack([x, y]), return_gap=True)
    assert np.array_equal(gaps, [1.0, 0.0])
    q = np.concatenate([np.repeat(x, 8, axis=0), np.repeat(y, 8, axis=0)])[None]     # 2 groups of 64
    k = rng.standard_normal((1, 128, 5))
    A, g = O.ibcs_scores(q, k, 64, qn=64, return_gap=True)
    # each group of 64 holds 8 copies of each of its rows: rows 0, 8, ..., 56 are the
    # initial centroids, all distinct in the first group (margin 1) and tied in the second
    assert np.array_equal(g[0], [1.0, 0.0])


def pin_ibcs_rows_and_threshold():
    rng = _rng(43)
    G, L, N, d = 2, 384, 64, 8
    q, k = (rng.standard_normal((G, L, d)).astype(np.float32) for _ in range(2))
    A = O.ibcs_scores(q, k, N)
    assert np.max(np.abs(A.sum(-1) - 1.0)) <= 1e-12 and np.all(A > 0)
    r0 = O.ibcs_block_mask(q, k, N, 0.0)
    assert r0["mask"].all()
    r = O.ibcs_block_mask(q, k, N, 0.3)
    # kept mass >= 1 - thr, and the row's largest score is kept
    kept_mass = np.where(r["mask"], r["A"], 0).sum(-1)
    assert np.all(kept_mass >= 0.7 - 1e-6)
    assert np.all(np.take_along_axis(r["mask"], np.argmax(r["A"], -1)[..., None], -1))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
