"""Comparison helpers for the GPU parity tests (GPU results vs the oracle)."""
from __future__ import annotations

import numpy as np

BAND = 1e-4          # |F_oracle - thr| within which a mask disagreement is tolerated
MAX_BAND_FRAC = 1e-3  # tolerated disagreements, as a fraction of all blocks
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def lists_to_mask(count: np.ndarray, index: np.ndarray) -> np.ndarray:
    """[..., nb] counts + [..., nb, nb] lists -> bool mask; also checks each list is
    ascending, unique and in range."""
    nb = index.shape[-1]
    c2 = count.reshape(-1).astype(np.int64)
    i2 = index.reshape(-1, nb)
    assert np.all((c2 >= 0) & (c2 <= nb)), "count out of range"
    valid = np.arange(nb)[None, :] < c2[:, None]
    vals = np.where(valid, i2, 0)
    assert np.all((vals >= 0) & (vals < nb)), "index out of range"
    d = np.diff(vals, axis=1)
    assert np.all((d > 0) | ~valid[:, 1:]), "lists must be strictly ascending"
    rows, cols = np.nonzero(valid)
    m = np.zeros((c2.size, nb), dtype=bool)
    m[rows, i2[rows, cols]] = True
    return m.reshape(index.shape)


def bitmap_to_mask(bitmap: np.ndarray, nb: int) -> np.ndarray:
    words = bitmap.astype(np.uint32)
    bits = (words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    flat = bits.reshape(bits.shape[:-2] + (-1,)).astype(bool)
    assert not flat[..., nb:].any(), "bits past nb must be zero"
    return flat[..., :nb]


TIE_EPS = 2e-5      # relative spread of pooled probabilities treated as a near tie


def cutoff_ambiguity(A: np.ndarray, thr: float, eps: float = TIE_EPS) -> np.ndarray:
    """Blocks whose keep bit float32 arithmetic cannot settle.

    F_j = (mass of blocks <= A_j) is only known up to the order of blocks whose
    values agree with A_j to within relative ``eps`` (about 5x the float32 error of
    the pooled softmax): over those orders F_j ranges from
        F_lo = mass of blocks < A_j (1 - eps), plus A_j
        F_hi = mass of blocks <= A_j (1 + eps).
    A block is at the cutoff when thr lies within BAND of [F_lo, F_hi].  Without
    near ties F_lo = F_hi = F_j and this is |F_j - thr| <= BAND."""
    nb = A.shape[-1]
    a = np.asarray(A, dtype=np.float64).reshape(-1, nb)
    f_lo = np.empty_like(a)
    f_hi = np.empty_like(a)
    for r in range(a.shape[0]):
        s = np.sort(a[r])
        c = np.concatenate([[0.0], np.cumsum(s)])      # c[n] = mass of the n smallest
        f_hi[r] = c[np.searchsorted(s, a[r] * (1 + eps), side="right")]
        f_lo[r] = c[np.searchsorted(s, a[r] * (1 - eps), side="left")] + a[r]
    amb = (thr >= f_lo - BAND) & (thr <= f_hi + BAND)
    return amb.reshape(A.shape)


def check_mask(gpu_mask: np.ndarray, oracle_mask: np.ndarray, oracle_A: np.ndarray, thr: float,
               oracle_F: np.ndarray = None, counts: dict = None):
    """Bit-exact except blocks at the cutoff (see cutoff_ambiguity), and those at most
    MAX_BAND_FRAC of all blocks.  Returns (mismatches, band population).

    With the oracle's F, the mismatches are also split into those the plain band
    |F - thr| <= BAND admits and those only the near-tie extension admits; the plain
    ones must stay within MAX_BAND_FRAC on their own.  ``counts`` (a dict) accumulates
    blocks, mismatches, plain, tie_only and band."""
    assert gpu_mask.shape == oracle_mask.shape
    mism = gpu_mask != oracle_mask
    in_band = cutoff_ambiguity(oracle_A, thr)
    outside = mism & ~in_band
    assert not outside.any(), (
        f"{int(outside.sum())} mask disagreements outside the band, e.g. at "
        f"{np.argwhere(outside)[:5].tolist()}")
    assert mism.sum() <= MAX_BAND_FRAC * mism.size, f"{int(mism.sum())} band disagreements"
    if oracle_F is not None:
        plain = mism & (np.abs(np.asarray(oracle_F, dtype=np.float64) - thr) <= BAND)
        assert plain.sum() <= MAX_BAND_FRAC * mism.size, f"{int(plain.sum())} plain-band disagreements"
        if counts is not None:
            counts["plain"] = counts.get("plain", 0) + int(plain.sum())
            counts["tie_only"] = counts.get("tie_only", 0) + int((mism & ~plain).sum())
    if counts is not None:
        counts["blocks"] = counts.get("blocks", 0) + int(mism.size)
        counts["mismatches"] = counts.get("mismatches", 0) + int(mism.sum())
        counts["band"] = counts.get("band", 0) + int(in_band.sum())
    return int(mism.sum()), int(in_band.sum())


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
