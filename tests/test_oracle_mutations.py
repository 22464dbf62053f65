"""Planted mistakes in the oracle (CPU only): each must make at least one pin fail.

This shows the pins are strong enough that a plausible slip (a dropped term, a
wrong sign or index, a transposed operand) in any oracle step would be caught."""
import numpy as np
import pytest

import oracle.nabla_oracle as O
import oracle_pins

_orig_fractal = O.fractal_index
_orig_pooled = O.pooled_logits
_orig_cdf = O.cdf_values


def _fractal_colmajor(T, H, W, P):
    # patches taken column-major inside each frame
    nH, nW = H // P, W // P
    pi = _orig_fractal(T, H, W, P)
    out = pi.copy()
    for l in range(T * H * W):
        t, rem = divmod(l, H * W)
        y, x = divmod(rem, W)
        patch = (t * nW + x // P) * nH + y // P
        out[l] = patch * P * P + (y % P) * P + (x % P)
    return out


def _pooled_transposed(qp, kp, scale, dtype=np.float32):
    return _orig_pooled(kp, qp, scale, dtype)


def _pooled_unscaled(qp, kp, scale, dtype=np.float32):
    return _orig_pooled(qp, kp, 1.0, dtype)


def _softmax_sign(S):
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(m - S)
    return e / np.sum(e, axis=-1, keepdims=True)


def _cdf_untied(A):
    # ties broken by position instead of grouped
    n = A.shape[-1]
    A2 = A.reshape(-1, n)
    order = np.argsort(A2, axis=1, kind="stable")
    c = np.cumsum(np.take_along_axis(A2, order, 1), axis=1, dtype=A.dtype)
    F = np.empty_like(c)
    np.put_along_axis(F, order, c, 1)
    return F.reshape(A.shape)


def _cdf_descending(A):
    # accumulates from the top instead of from the bottom
    return (1.0 - _orig_cdf(A) + A).astype(A.dtype)


def _keep_nonstrict(A, thr):
    F = O.cdf_values(A)
    return F >= F.dtype.type(thr)


def _block_mean_off_by_one(x, N, dtype=np.float32):
    L, d = x.shape[-2], x.shape[-1]
    xb = np.asarray(x, dtype=dtype).reshape(x.shape[:-2] + (L // N, N, d))
    return xb[..., 1:, :].sum(-2) / dtype(N)       # drops the first token of each block


def _sta_strict(T, H, W, P, N, window):
    r = np.array([(w - 1) // 2 for w in window])
    tiles = O.block_tiles(T, H, W, P, N)
    return np.all(np.abs(tiles[:, None] - tiles[None]) < np.maximum(r, 1), axis=-1)


def _attn_no_scale(q, k, v, keep, i, N, scale, dtype=np.float64):
    js = np.nonzero(keep)[0]
    tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
    s = np.asarray(q[i * N:(i + 1) * N], dtype) @ np.asarray(k[tok], dtype).T
    p = np.exp(s - s.max(1, keepdims=True))
    return (p @ np.asarray(v[tok], dtype)) / p.sum(1, keepdims=True)


def _attn_keys_shifted(q, k, v, keep, i, N, scale, dtype=np.float64):
    js = np.nonzero(keep)[0]
    tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
    tok_v = (tok + 1) % k.shape[0]                     # V rows one token off
    s = (np.asarray(q[i * N:(i + 1) * N], dtype) @ np.asarray(k[tok], dtype).T) * scale
    p = np.exp(s - s.max(1, keepdims=True))
    return (p @ np.asarray(v[tok_v], dtype)) / p.sum(1, keepdims=True)


def _backward_with(bug):
    """A copy of the oracle's backward with one planted slip."""
    def bwd(q, k, v, dout, mask, N, scale=None, dtype=np.float64):
        d = q.shape[-1]
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        G, L, _ = q.shape
        dq, dk, dv = (np.zeros((G, L, d), dtype=dtype) for _ in range(3))
        for g in range(G):
            for i in range(L // N):
                js = np.nonzero(mask[g, i])[0]
                if len(js) == 0:
                    continue
                tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
                rows = slice(i * N, (i + 1) * N)
                qi, kk, vv, doi = (np.asarray(a, dtype) for a in (q[g, rows], k[g, tok], v[g, tok], dout[g, rows]))
                s = (qi @ kk.T) * scale
                e = np.exp(s - s.max(1, keepdims=True))
                p = e / e.sum(1, keepdims=True)
                D = np.sum(doi * (p @ vv), axis=1, keepdims=True)
                dP = doi @ vv.T
                ds = p * dP if bug == "no_D" else p * (dP - D)
                dv[g, tok] += (p.T @ doi) if bug != "dv_from_dp" else (ds.T @ doi)
                dq[g, rows] = (ds @ kk) * (1.0 if bug == "dq_unscaled" else scale)
                dk[g, tok] += scale * ((ds.T @ qi) if bug != "dk_from_p" else (p.T @ qi))
        return dq, dk, dv
    bwd.__name__ = f"_backward_{bug}"
    return bwd


def _lse_log2(q, k, keep, i, N, scale, dtype=np.float64):
    return _orig_block_lse(q, k, keep, i, N, scale, dtype) / np.log(2.0)


_orig_block_lse = O.block_lse
_orig_sip_p = O.sip_probabilities
_orig_sip_mask = O.sip_mask
_orig_wattn = O.weighted_block_attention


def _sip_uncapped(A, budget):
    # proportional allocation without the cap at 1 (and no certain blocks)
    A = np.asarray(A, dtype=np.float64)
    if budget >= len(A):
        return np.ones(len(A))
    return np.minimum(budget * A / A.sum(), 1.5)


def _sip_no_certain_top(A, budget):
    p = _orig_sip_p(A, budget).copy()
    t = int(np.argmax(A))
    if budget < len(A):
        p[t] = min(1.0, p[t] * 0.5)
    return p


def _sip_logw_sign(A, budget, uniforms):
    m, logw, pi = _orig_sip_mask(A, budget, uniforms)
    return m, -logw, pi


def _wattn_shift_ignored(q, k, v, mask, logw, N, scale=None, dtype=np.float64):
    return _orig_wattn(q, k, v, mask, np.zeros_like(logw), N, scale, dtype)

_orig_ibcs_clusters = O.ibcs_clusters
_orig_ibcs_scores = O.ibcs_scores


def _ibcs_uniform_weights(qblock, n_clusters=8, iters=4):
    cent, w = _orig_ibcs_clusters(qblock, n_clusters, iters)
    return cent, np.full(n_clusters, 1.0 / n_clusters)


def _ibcs_first_rows_init(qblock, n_clusters=8, iters=4):
    # initial centroids from the first k rows instead of evenly spaced ones
    x = np.asarray(qblock, dtype=np.float32)
    y = x.copy()
    idx = np.arange(n_clusters) * (len(x) // n_clusters)
    y[idx], y[np.arange(n_clusters)] = x[np.arange(n_clusters)], x[idx]
    return _orig_ibcs_clusters(y, n_clusters, iters)


def _ibcs_softmax_over_centroids(q, k, N, scale=None):
    A = _orig_ibcs_scores(q, k, N, scale)
    return np.exp(A) / np.exp(A).sum(-1, keepdims=True)


def _ibcs_group_ignored(q, k, N, scale=None, qn=None):
    # every 64-token block clustered on its own, whatever the group size
    return _orig_ibcs_scores(q, k, N, scale)


_orig_block_mask = O.block_mask


def _block_mask_and(q, k, T, H, W, P, N, thr, sta=None, scale=None, dtype=np.float32):
    # the window intersected with the CDF mask instead of joined to it
    res = _orig_block_mask(q, k, T, H, W, P, N, thr, None, scale, dtype)
    if sta is not None:
        res["mask"] = res["mask_nabla"] & O.sta_mask(T, H, W, P, N, sta)
    return res


def _ibcs_gap_unscaled(qgroup, n_clusters=8, iters=4, return_gap=False):
    # the margin taken as an absolute difference, not relative to the distance
    out = _orig_ibcs_clusters(qgroup, n_clusters, iters, return_gap=True)
    if not return_gap:
        return out[:2]
    x = np.asarray(qgroup, dtype=np.float64)
    return out[0], out[1], out[2] * float(np.sum(x[..., :1, :] ** 2) + 1.0)


def _ibcs_last_round_weights_off(qgroup, n_clusters=8, iters=4, return_gap=False):
    # weights from the assignment one round earlier than the centroids' last update
    out = _orig_ibcs_clusters(qgroup, n_clusters, max(iters - 1, 1), return_gap=True)
    cent = _orig_ibcs_clusters(qgroup, n_clusters, iters)[0]
    res = (cent, out[1], out[2])
    return res if return_gap else res[:2]


MUTATIONS = [
    ("fractal_index", _fractal_colmajor),
    ("pooled_logits", _pooled_transposed),
    ("pooled_logits", _pooled_unscaled),
    ("row_softmax", _softmax_sign),
    ("cdf_values", _cdf_untied),
    ("cdf_values", _cdf_descending),
    ("cdf_keep", _keep_nonstrict),
    ("block_mean", _block_mean_off_by_one),
    ("sta_mask", _sta_strict),
    ("attention_block", _attn_no_scale),
    ("attention_block", _attn_keys_shifted),
    ("masked_attention_backward", _backward_with("no_D")),
    ("masked_attention_backward", _backward_with("dv_from_dp")),
    ("masked_attention_backward", _backward_with("dq_unscaled")),
    ("masked_attention_backward", _backward_with("dk_from_p")),
    ("block_lse", _lse_log2),
    ("sip_probabilities", _sip_uncapped),
    ("sip_probabilities", _sip_no_certain_top),
    ("sip_mask", _sip_logw_sign),
    ("weighted_block_attention", _wattn_shift_ignored),
    ("ibcs_clusters", _ibcs_uniform_weights),
    ("ibcs_clusters", _ibcs_first_rows_init),
    ("ibcs_scores", _ibcs_softmax_over_centroids),
    ("ibcs_scores", _ibcs_group_ignored),
    ("block_mask", _block_mask_and),
    ("ibcs_clusters", _ibcs_gap_unscaled),
    ("ibcs_clusters", _ibcs_last_round_weights_off),
]


@pytest.mark.parametrize("name,bug", MUTATIONS, ids=[f"{n}:{b.__name__}" for n, b in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, bug):
    monkeypatch.setattr(O, name, bug)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
