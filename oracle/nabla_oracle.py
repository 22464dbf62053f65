"""Oracle for NABLA block-mean adaptive block-sparse attention (forward, and the
gradient of its attention step).

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow CPU statement of what the
GPU path computes.  Only the test suite, the smoke check and the bench's CPU
baseline may import it; the library and its Python binding never do, and the two
share no code.  Everything here is numpy (plus torch's CPU bf16 cast inside the
input generator, which lives elsewhere).

Source: the technical summary "NABLA - Atenção de Bloco Adaptativa de Vizinhança
para Geração de Vídeo Eficiente" (gist.science, paper 2507.13546), sections
"Declaração do Problema" and "Metodologia: NABLA" (items 1-3), plus the
AB-Attention news page, section "Onde os esquemas esparsos anteriores falham"
(a dropped block leaves both the numerator and the softmax normaliser).

Precision.  The mask steps (pooling, pooled map, softmax, cumulative mass) run in
float32 by default: they turn floating point into a keep/drop bit, and the GPU
takes that decision in float32.  Masked attention runs in float64.  Every
function takes a ``dtype`` so a test can rerun a step in float64.

Readings of the pages (they leave these open):
  * raster flatten l = (t*H + y)*W + x; non-causal self-attention; scale 1/sqrt(d);
  * "fractal flattening" = row-major order of P x P patches per frame, row-major
    inside a patch, frames kept in order;
  * the garbled "average pooling in N x N blocks" = mean of N consecutive
    reordered tokens of Q and of K (equal to the tile mean of the logits by
    bilinearity);
  * the reduced map is row-softmaxed with the same scale as the attention;
  * "keep the blocks whose accumulated probability exceeds 1 - thr" = the
    nucleus rule: with F_ij = sum of A_ik over k with A_ik <= A_ij (tied blocks
    grouped), keep iff F_ij > thr, so thr = 0 keeps every block;
  * the STA window is centred on the query tile (1 frame x P x P patch) and
    truncated at the grid border; the final mask is the OR of both masks;
  * kept KV blocks are listed in ascending block order.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Step 1: token reordering ("fractal flattening", Metodologia item 1)
# ---------------------------------------------------------------------------

def fractal_index(T: int, H: int, W: int, P: int) -> np.ndarray:
    """pi[l] = position in fractal order of the raster token l = (t*H + y)*W + x.

    Frames stay in time order; inside a frame the P x P patches are taken
    row-major and each patch's P*P tokens are made contiguous (row-major inside
    the patch)."""
    if H % P or W % P:
        raise ValueError("H and W must be multiples of P")
    nH, nW = H // P, W // P
    pi = np.empty(T * H * W, dtype=np.int64)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                l = (t * H + y) * W + x
                patch = (t * nH + y // P) * nW + x // P
                pi[l] = patch * P * P + (y % P) * P + (x % P)
    return pi


def reorder(x: np.ndarray, T: int, H: int, W: int, P: int, inverse: bool = False) -> np.ndarray:
    """Move the token axis (-2) of ``x`` from raster to fractal order, or back."""
    pi = fractal_index(T, H, W, P)
    out = np.empty_like(x)
    if not inverse:
        out[..., pi, :] = x
    else:
        out[...] = x[..., pi, :]
    return out


# ---------------------------------------------------------------------------
# Step 2: adaptive mask (Metodologia item 2)
# ---------------------------------------------------------------------------

def block_mean(x: np.ndarray, N: int, dtype=np.float32) -> np.ndarray:
    """Mean of each run of N consecutive tokens (axis -2): [..., L, d] -> [..., L/N, d].

    Summed one token at a time, in token order, in ``dtype``."""
    L, d = x.shape[-2], x.shape[-1]
    if L % N:
        raise ValueError("L must be a multiple of N")
    xb = np.asarray(x, dtype=dtype).reshape(x.shape[:-2] + (L // N, N, d))
    acc = np.zeros(x.shape[:-2] + (L // N, d), dtype=dtype)
    for r in range(N):
        acc += xb[..., r, :]
    return acc / dtype(N)


def pooled_logits(qp: np.ndarray, kp: np.ndarray, scale: float, dtype=np.float32) -> np.ndarray:
    """S = Qp Kp^T * scale, the reduced attention map before the softmax."""
    qp = np.asarray(qp, dtype=dtype)
    kp = np.asarray(kp, dtype=dtype)
    return np.matmul(qp, np.swapaxes(kp, -1, -2)) * dtype(scale)


def row_softmax(S: np.ndarray) -> np.ndarray:
    """A_ij = exp(S_ij - max_k S_ik) / sum_k exp(S_ik - max_k S_ik), in S's dtype."""
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def cdf_values(A: np.ndarray) -> np.ndarray:
    """F_ij = sum over k with A_ik <= A_ij of A_ik (the row's cumulative mass at A_ij).

    Computed by a stable ascending sort and a sequential running sum; every
    member of a run of equal values takes the running sum at the run's end, so
    tied blocks share one F."""
    A = np.asarray(A)
    n = A.shape[-1]
    A2 = A.reshape(-1, n)
    order = np.argsort(A2, axis=1, kind="stable")
    s = np.take_along_axis(A2, order, axis=1)
    c = np.cumsum(s, axis=1, dtype=A.dtype)
    pos = np.broadcast_to(np.arange(n), s.shape)
    run_end = np.ones(s.shape, dtype=bool)
    run_end[:, :-1] = s[:, 1:] != s[:, :-1]
    last = np.where(run_end, pos, n)
    last = np.minimum.accumulate(last[:, ::-1], axis=1)[:, ::-1]
    Fs = np.take_along_axis(c, last, axis=1)
    F = np.empty_like(Fs)
    np.put_along_axis(F, order, Fs, axis=1)
    return F.reshape(A.shape)


def cdf_keep(A: np.ndarray, thr: float) -> np.ndarray:
    """Keep bit of each block: F_ij > thr (the mass that may be dropped is <= thr)."""
    if not (0.0 <= thr < 1.0):
        raise ValueError("thr must lie in [0, 1)")
    F = cdf_values(A)
    return F > F.dtype.type(thr)


# ---------------------------------------------------------------------------
# Step 3: static Sliding Tile window (Metodologia item 3)
# ---------------------------------------------------------------------------

def block_tiles(T: int, H: int, W: int, P: int, N: int) -> np.ndarray:
    """(t, patch row, patch column) of every N-token block of the fractal order,
    read off the raster coordinates of the tokens it holds.  Needs N == P*P so a
    block is exactly one 1 x P x P tile."""
    if N != P * P:
        raise ValueError("a tile is one frame x one P x P patch, so N must equal P*P")
    pi = fractal_index(T, H, W, P)
    L = T * H * W
    l_of = np.empty(L, dtype=np.int64)
    l_of[pi] = np.arange(L)
    nb = L // N
    tiles = np.empty((nb, 3), dtype=np.int64)
    for i in range(nb):
        ls = l_of[i * N:(i + 1) * N]
        t, rem = np.divmod(ls, H * W)
        y, x = np.divmod(rem, W)
        coords = {(int(a), int(b) // P, int(c) // P) for a, b, c in zip(t, y, x)}
        if len(coords) != 1:
            raise AssertionError("block straddles tiles")
        tiles[i] = coords.pop()
    return tiles


def sta_mask(T: int, H: int, W: int, P: int, N: int, window: Tuple[int, int, int]) -> np.ndarray:
    """M_STA[i, j]: tile of block j lies inside the window centred on block i's tile
    (|dt| <= rt, |dh| <= rh, |dw| <= rw, r = (w - 1) / 2), truncated at the border."""
    wt, wh, ww = window
    if min(window) <= 0 or wt % 2 == 0 or wh % 2 == 0 or ww % 2 == 0:
        raise ValueError("STA window sizes must be odd and positive")
    r = np.array([(wt - 1) // 2, (wh - 1) // 2, (ww - 1) // 2])
    tiles = block_tiles(T, H, W, P, N)
    diff = np.abs(tiles[:, None, :] - tiles[None, :, :])
    return np.all(diff <= r, axis=-1)


# ---------------------------------------------------------------------------
# Mask assembly and expansion into kept-KV lists
# ---------------------------------------------------------------------------

def block_mask(q: np.ndarray, k: np.ndarray, T: int, H: int, W: int, P: int, N: int,
               thr: float, sta: Optional[Tuple[int, int, int]] = None,
               scale: Optional[float] = None, dtype=np.float32) -> Dict[str, np.ndarray]:
    """Block mask for Q, K already in fractal order ([..., L, d]).

    Returns ``mask`` (final, [..., nb, nb] bool), ``mask_nabla`` (CDF part only),
    ``F`` (cumulative mass), ``A`` (pooled softmax) and ``S`` (pooled logits)."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qp = block_mean(q, N, dtype)
    kp = block_mean(k, N, dtype)
    S = pooled_logits(qp, kp, scale, dtype)
    A = row_softmax(S)
    F = cdf_values(A)
    m_nabla = F > F.dtype.type(thr)
    m = m_nabla
    if sta is not None:
        m = m_nabla | sta_mask(T, H, W, P, N, sta)
    return {"mask": m, "mask_nabla": m_nabla, "F": F, "A": A, "S": S}


def kv_lists(mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per query block, the count and the ascending list of kept KV blocks.

    ``index`` is [..., nb, nb] int32 with entries past the count set to -1."""
    nb = mask.shape[-1]
    m2 = mask.reshape(-1, nb, nb)
    count = m2.sum(axis=-1).astype(np.int32)
    index = np.full(m2.shape, -1, dtype=np.int32)
    for r in range(m2.shape[0]):
        for i in range(nb):
            js = np.nonzero(m2[r, i])[0]
            index[r, i, :len(js)] = js
    return count.reshape(mask.shape[:-1]), index.reshape(mask.shape)


def mask_from_lists(count: np.ndarray, index: np.ndarray) -> np.ndarray:
    """Inverse of :func:`kv_lists` (entries past each count are ignored)."""
    nb = index.shape[-1]
    c2 = np.asarray(count).reshape(-1, nb)
    i2 = np.asarray(index).reshape(-1, nb, nb)
    m = np.zeros(i2.shape, dtype=bool)
    for r in range(i2.shape[0]):
        for i in range(nb):
            c = int(c2[r, i])
            m[r, i, i2[r, i, :c]] = True
    return m.reshape(np.asarray(index).shape)


# ---------------------------------------------------------------------------
# Block-sparse attention = softmax attention with masked tiles removed
# ---------------------------------------------------------------------------

def attention_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray, i: int,
                    N: int, scale: float, dtype=np.float64) -> np.ndarray:
    """Output rows of query block ``i`` of one head ([L, d] inputs, fractal order).

    Softmax attention of the block's N queries over the keys of the kept blocks
    ``keep`` (bool [nb]); a dropped block contributes to neither the numerator nor
    the normaliser.  Two passes: row max, then exp and sum.  A query block with
    no kept block returns zeros."""
    js = np.nonzero(keep)[0]
    if len(js) == 0:
        return np.zeros((N, q.shape[-1]), dtype=dtype)
    tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
    qi = np.asarray(q[i * N:(i + 1) * N], dtype=dtype)
    kk = np.asarray(k[tok], dtype=dtype)
    vv = np.asarray(v[tok], dtype=dtype)
    s = (qi @ kk.T) * dtype(scale)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ vv) / np.sum(p, axis=1, keepdims=True)


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, N: int,
                     scale: Optional[float] = None, dtype=np.float64,
                     blocks: Optional[Iterable[Tuple[int, int]]] = None):
    """O = block-masked softmax attention for [G, L, d] inputs and a [G, nb, nb] mask.

    Without ``blocks`` the whole [G, L, d] output is returned; with a list of
    (g, i) pairs only those query blocks are computed and a dict maps each pair
    to its [N, d] rows (rows are independent given the mask)."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    if blocks is not None:
        return {(g, i): attention_block(q[g], k[g], v[g], mask[g, i], i, N, scale, dtype)
                for g, i in blocks}
    G, L, _ = q.shape
    out = np.empty((G, L, v.shape[-1]), dtype=dtype)
    for g in range(G):
        for i in range(L // N):
            out[g, i * N:(i + 1) * N] = attention_block(q[g], k[g], v[g], mask[g, i], i, N,
                                                        scale, dtype)
    return out


def block_lse(q: np.ndarray, k: np.ndarray, keep: np.ndarray, i: int, N: int, scale: float,
              dtype=np.float64) -> np.ndarray:
    """Natural-log log-sum-exp of the kept logits of each query row of block ``i``:
    lse_a = log sum over kept keys b of exp(scale * q_a . k_b); -inf for a block with
    no kept KV block.  Row max first, then the sum of exponentials."""
    js = np.nonzero(keep)[0]
    if len(js) == 0:
        return np.full(N, -np.inf, dtype=dtype)
    tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
    s = (np.asarray(q[i * N:(i + 1) * N], dtype=dtype) @ np.asarray(k[tok], dtype=dtype).T) * dtype(scale)
    m = np.max(s, axis=1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def masked_attention_lse(q: np.ndarray, k: np.ndarray, mask: np.ndarray, N: int,
                         scale: Optional[float] = None, dtype=np.float64) -> np.ndarray:
    """[G, L] log-sum-exp of every query row over its kept keys (see ``block_lse``)."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    G, L, _ = q.shape
    out = np.empty((G, L), dtype=dtype)
    for g in range(G):
        for i in range(L // N):
            out[g, i * N:(i + 1) * N] = block_lse(q[g], k[g], mask[g, i], i, N, scale, dtype)
    return out


def masked_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                              mask: np.ndarray, N: int, scale: Optional[float] = None,
                              dtype=np.float64):
    """Gradients (dq, dk, dv) of sum(O * dout) for O = block-masked softmax attention
    (``masked_attention``) of [G, L, d] inputs under a [G, nb, nb] mask.

    The pages define the forward only; this is its gradient, written per query block
    i over the tokens of its kept KV blocks:
        P   = softmax of scale * Q_i K^T over the kept keys (row by row)
        O_i = P V,   D = rowsum(dO_i * O_i)
        dV  += P^T dO_i,   dP = dO_i V^T,   dS = P * (dP - D)
        dQ_i = scale * dS K,   dK += scale * dS^T Q_i
    A query block with no kept block has zero output, so it passes no gradient."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    G, L, _ = q.shape
    dq = np.zeros((G, L, d), dtype=dtype)
    dk = np.zeros((G, L, d), dtype=dtype)
    dv = np.zeros((G, L, v.shape[-1]), dtype=dtype)
    for g in range(G):
        for i in range(L // N):
            js = np.nonzero(mask[g, i])[0]
            if len(js) == 0:
                continue
            tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
            rows = slice(i * N, (i + 1) * N)
            qi = np.asarray(q[g, rows], dtype=dtype)
            kk = np.asarray(k[g, tok], dtype=dtype)
            vv = np.asarray(v[g, tok], dtype=dtype)
            doi = np.asarray(dout[g, rows], dtype=dtype)
            s = (qi @ kk.T) * dtype(scale)
            e = np.exp(s - np.max(s, axis=1, keepdims=True))
            p = e / np.sum(e, axis=1, keepdims=True)
            o = p @ vv
            D = np.sum(doi * o, axis=1, keepdims=True)
            dv[g, tok] += p.T @ doi
            ds = p * (doi @ vv.T - D)
            dq[g, rows] = dtype(scale) * (ds @ kk)
            dk[g, tok] += dtype(scale) * (ds.T @ qi)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# IBCS: intra-block clustering selector (AB-Attention page, "Os três recursos do
# AB-Attention", first feature) as an alternative block score for NABLA's CDF cut
# ---------------------------------------------------------------------------

IBCS_CLUSTERS = 8
IBCS_ITERS = 4


IBCS_TIE_EPS = 1e-5


def ibcs_clusters(qgroup: np.ndarray, n_clusters: int = IBCS_CLUSTERS, iters: int = IBCS_ITERS,
                  return_gap: bool = False):
    """Lloyd's k-means of one group of n queries ([n, d]), or of a batch of groups
    ([G, n, d]), into n_clusters clusters each, in float64.

    Readings (the page gives the cluster count, not the algorithm's steps): the initial
    centroids are the queries at rows 0, n/k, 2n/k, ...; ``iters`` rounds of
    assign-then-update; a query joins the centroid at the smallest squared Euclidean
    distance (ties to the lowest cluster index); a centroid moves to the mean of its
    queries, and an empty cluster keeps its centroid.  Returns (centroids [..., k, d],
    weights [..., k] = fraction of the group's queries in each cluster under the last
    assignment).

    With ``return_gap`` a third value gives, per group, the smallest relative margin
    (second-smallest minus smallest squared distance, over the second-smallest) of any
    query in any round.  An assignment whose margin is below a few float32 rounding
    errors of a d-term sum can come out either way in float32 arithmetic."""
    x = np.asarray(qgroup, dtype=np.float64)
    single = x.ndim == 2
    if single:
        x = x[None]
    G, n, d = x.shape
    k = n_clusters
    cent = x[:, np.arange(k) * (n // k)].copy()
    gap = np.full(G, np.inf)
    assign = np.zeros((G, n), dtype=np.int64)
    for _ in range(iters):
        dist = np.stack([np.sum((x - cent[:, c:c + 1, :]) ** 2, axis=-1) for c in range(k)], axis=-1)
        assign = np.argmin(dist, axis=-1)                    # first minimum: lowest index on ties
        two = np.sort(dist, axis=-1)[..., :2]
        margin = (two[..., 1] - two[..., 0]) / np.maximum(two[..., 1], np.finfo(np.float64).tiny)
        gap = np.minimum(gap, margin.min(axis=-1))
        for c in range(k):
            member = assign == c
            count = member.sum(axis=1)
            total = np.where(member[..., None], x, 0.0).sum(axis=1)
            has = count > 0
            cent[has, c] = total[has] / count[has][:, None]
    weights = np.stack([np.bincount(a, minlength=k) for a in assign]).astype(np.float64) / n
    out = (cent, weights, gap)
    if single:
        out = (cent[0], weights[0], gap[0])
    return out if return_gap else out[:2]


def ibcs_scores(q: np.ndarray, k: np.ndarray, N: int, scale: Optional[float] = None,
                qn: Optional[int] = None, return_gap: bool = False):
    """IBCS block scores for [..., L, d] Q, K in fractal order, in float64.

    The queries are taken in groups of qn consecutive tokens (default N; the page's
    setting is 128) and each group is clustered (ibcs_clusters).  With centroids mu_c and
    weights w_c of the group holding query block i,
        A_ij = sum_c w_c softmax_j(scale * mu_c . Kp_j),
    Kp_j the mean key of N-token block j: the weighted attention of the centroids to the
    mean keys.  The qn / N blocks of a group share one row.  Rows sum to one like NABLA's
    pooled softmax, so the same CDF cut applies.  With ``return_gap`` also the clustering
    margin of each row's group ([..., nb], see ibcs_clusters)."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    L = q.shape[-2]
    qn = N if qn is None else qn
    if qn % N or L % qn:
        raise ValueError("qn must be a multiple of N that divides L")
    nb = L // N
    per = qn // N
    lead = q.shape[:-2]
    qf = np.asarray(q, dtype=np.float64).reshape((-1, L, d))
    kp = block_mean(np.asarray(k).reshape((-1, L, d)), N, np.float64)
    A = np.zeros((qf.shape[0], nb, nb))
    gap = np.zeros((qf.shape[0], nb))
    for g in range(qf.shape[0]):
        cents, ws, gg = ibcs_clusters(qf[g].reshape(L // qn, qn, d), return_gap=True)   # every group of the head
        gap[g] = np.repeat(gg, per)
        for gi in range(L // qn):
            S = (cents[gi] @ kp[g].T) * scale                                    # [k, nb]
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            A[g, gi * per:(gi + 1) * per] = ws[gi] @ P
    A = A.reshape(lead + (nb, nb))
    return (A, gap.reshape(lead + (nb,))) if return_gap else A


def ibcs_block_mask(q: np.ndarray, k: np.ndarray, N: int, thr: float,
                    scale: Optional[float] = None, qn: Optional[int] = None) -> Dict[str, np.ndarray]:
    """NABLA's CDF cut on the IBCS scores: keep block j of row i iff the mass of the
    blocks scoring at most A_ij exceeds thr.  Returns mask, F, A (the scores rounded to
    float32, where the cut is taken) and gap (each row's clustering margin)."""
    A, gap = ibcs_scores(q, k, N, scale, qn, return_gap=True)
    A32 = A.astype(np.float32)
    F = cdf_values(A32)
    return {"mask": F > F.dtype.type(thr), "F": F, "A": A32, "gap": gap}


# ---------------------------------------------------------------------------
# SIP: sampling with inclusion-probability weighting (AB-Attention page, "Os três
# recursos do AB-Attention", second feature), on NABLA's block scores
# ---------------------------------------------------------------------------

def sip_probabilities(A: np.ndarray, budget: int) -> np.ndarray:
    """Inclusion probabilities of one row of block scores A (>= 0) for an expected
    budget of ``budget`` blocks: a block's probability is proportional to its score,
    capped at 1, and the highest-scoring block is always included.

    Reading: the row's top block (smallest index among equal maxima) gets pi = 1; the
    other blocks share budget - 1 by pi_j = min(1, c A_j) with c chosen so that their
    probabilities sum to budget - 1 (blocks whose c A_j reaches 1 are certain).  With
    budget >= nb every block is certain.  Solved by sorting the scores in decreasing
    order and taking the smallest number m of certain blocks for which the next block
    stays below 1."""
    A = np.asarray(A, dtype=np.float64)
    nb = A.shape[-1]
    pi = np.zeros(nb)
    if budget >= nb:
        return np.ones(nb)
    t = int(np.argmax(A))
    pi[t] = 1.0
    rest = np.array([j for j in range(nb) if j != t])
    kp = budget - 1
    if kp <= 0 or len(rest) == 0:
        return pi
    w = A[rest]
    order = np.argsort(-w, kind="stable")
    ws = w[order]
    tail = np.concatenate([np.cumsum(ws[::-1])[::-1], [0.0]])    # tail[m] = sum of ws[m:]
    c = 0.0
    m_cert = 0
    for m in range(0, min(kp, len(ws)) + 1):
        if m == kp or tail[m] <= 0.0:
            c, m_cert = 0.0, m
            break
        cm = (kp - m) / tail[m]
        if cm * ws[m] < 1.0:
            c, m_cert = cm, m
            break
    p_rest = np.minimum(1.0, c * ws)
    p_rest[:m_cert] = 1.0
    out = np.empty(len(rest))
    out[order] = p_rest
    pi[rest] = out
    return pi


def sip_mask(A: np.ndarray, budget: int, uniforms: np.ndarray):
    """Sampled mask and weights for rows of scores A [..., nb]: block j of a row is
    kept when its uniform draw u_j (in [0, 1), given) is below pi_j, and a kept block
    carries the logit shift log(1 / pi_j), so that exp(s + log(1/pi)) = exp(s) / pi:
    the Horvitz-Thompson weight of the sampled block in both the numerator and the
    normaliser of the softmax.  Returns (mask, logw, pi); logw is 0 where not kept."""
    A = np.asarray(A, dtype=np.float64)
    nb = A.shape[-1]
    flat = A.reshape(-1, nb)
    u = np.asarray(uniforms, dtype=np.float64).reshape(-1, nb)
    pi = np.stack([sip_probabilities(r, budget) for r in flat])
    keep = u < pi
    logw = np.where(keep, -np.log(np.where(keep, pi, 1.0)), 0.0)
    return keep.reshape(A.shape), logw.reshape(A.shape), pi.reshape(A.shape)


def weighted_block_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                             logw: np.ndarray, N: int, scale: Optional[float] = None,
                             dtype=np.float64) -> np.ndarray:
    """Block-sparse attention with a per-tile additive logit shift: for query block i,
    the logits of the tokens of kept KV block j are scale * q . k + logw[i, j]; dropped
    blocks are out of the numerator and the normaliser.  [G, L, d] inputs, [G, nb, nb]
    mask and shifts."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    G, L, _ = q.shape
    out = np.zeros((G, L, v.shape[-1]), dtype=dtype)
    for g in range(G):
        for i in range(L // N):
            js = np.nonzero(mask[g, i])[0]
            if len(js) == 0:
                continue
            tok = (js[:, None] * N + np.arange(N)[None, :]).reshape(-1)
            s = (np.asarray(q[g, i * N:(i + 1) * N], dtype) @ np.asarray(k[g, tok], dtype).T) * dtype(scale)
            s = s + np.repeat(np.asarray(logw[g, i, js], dtype), N)[None, :]
            e = np.exp(s - np.max(s, axis=1, keepdims=True))
            out[g, i * N:(i + 1) * N] = (e @ np.asarray(v[g, tok], dtype)) / np.sum(e, axis=1, keepdims=True)
    return out


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: int, H: int, W: int, P: int,
            N: int, thr: float, sta: Optional[Tuple[int, int, int]] = None,
            scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Whole path for raster-order [G, L, d] inputs: reorder, mask, attention and
    the inverse reorder of the output (returned in raster order)."""
    qf = reorder(q, T, H, W, P)
    kf = reorder(k, T, H, W, P)
    vf = reorder(v, T, H, W, P)
    mk = block_mask(qf, kf, T, H, W, P, N, thr, sta, scale)
    of = masked_attention(qf, kf, vf, mk["mask"], N, scale)
    mk["out"] = reorder(of, T, H, W, P, inverse=True)
    return mk
