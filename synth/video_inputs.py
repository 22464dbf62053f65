"""Seeded smooth-field + noise Q/K/V for a T x H x W latent video grid.

Recipe (one (b, h) pair at a time, raster token order l = (t*H + y)*W + x):

* ``SeedSequence([seed, b, h]).spawn(5)`` gives five independent streams: the
  shared Q/K field, the V field, and the Q, K, V noise.
* A field is a sum of 8 cosines over (t, y, x) with integer wave numbers
  k_t in {0,1,2}, k_h, k_w in {0..3} and a random phase per (cosine, channel);
  each cosine has amplitude 0.5, so every channel has unit RMS.
* Q and K share one field (independent noise), so q.k peaks at small
  space-time distance, the decay of attention with distance that the Radial
  Attention article describes; V has its own field.  Noise is N(0, 0.5^2).
* Optionally Q and K are scaled by s with s^2 = 8 sqrt(d) / mean_l(q_l . k_l),
  so the diagonal logits q.k/sqrt(d) average 8 and random pairs span about +-5.
* Values are rounded once to the workload dtype (bf16 RNE); both the oracle
  and the GPU consume the rounded values.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np
import torch

from .configs import Config

GENERATOR_VERSION = "cosfield-v1"

_N_COS = 8


def _field(rng: np.random.Generator, T: int, H: int, W: int, d: int) -> np.ndarray:
    kt = rng.integers(0, 3, size=_N_COS)
    kh = rng.integers(0, 4, size=_N_COS)
    kw = rng.integers(0, 4, size=_N_COS)
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(_N_COS, d))
    t = np.arange(T, dtype=np.float64)[:, None, None, None]
    y = np.arange(H, dtype=np.float64)[None, :, None, None]
    x = np.arange(W, dtype=np.float64)[None, None, :, None]
    theta = 2.0 * np.pi * (kt * t / T + kh * y / H + kw * x / W)     # [T,H,W,8]
    theta = theta.reshape(T * H * W, _N_COS)
    # cos(theta + phi) = cos(theta)cos(phi) - sin(theta)sin(phi), as two small matmuls
    f = 0.5 * (np.cos(theta) @ np.cos(phase) - np.sin(theta) @ np.sin(phase))
    return f.astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    return x.astype(np.float32)


def make_head(cfg: Config, b: int, h: int, seed: Optional[int] = None
              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of one (b, h) pair as float32 arrays [L, d] in raster order,
    already rounded to the workload dtype."""
    seed = cfg.index if seed is None else seed
    ss = np.random.SeedSequence([seed, b, h])
    s_fqk, s_fv, s_nq, s_nk, s_nv = (np.random.default_rng(c) for c in ss.spawn(5))
    L, d = cfg.L, cfg.d
    fqk = _field(s_fqk, cfg.T, cfg.H, cfg.W, d)
    fv = _field(s_fv, cfg.T, cfg.H, cfg.W, d)
    q = fqk + 0.5 * s_nq.standard_normal((L, d), dtype=np.float32)
    k = fqk + 0.5 * s_nk.standard_normal((L, d), dtype=np.float32)
    v = fv + 0.5 * s_nv.standard_normal((L, d), dtype=np.float32)
    if cfg.scale_logits:
        mean_qk = float(np.mean(np.einsum("ld,ld->l", q.astype(np.float64), k.astype(np.float64))))
        s = np.float32(np.sqrt(8.0 * np.sqrt(d) / mean_qk))
        q = q * s
        k = k * s
    return _round(q, cfg.dtype), _round(k, cfg.dtype), _round(v, cfg.dtype)


def make_qkv(cfg: Config, seed: Optional[int] = None,
             pairs: Optional[Iterable[Tuple[int, int]]] = None):
    """Q, K, V torch CPU tensors [B, heads, L, d] in the workload dtype, raster order.

    With ``pairs`` only those (b, h) slices are filled (the rest stay zero);
    that keeps sampled checks at the largest shapes cheap."""
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = (cfg.B, cfg.heads, cfg.L, cfg.d)
    out = [torch.zeros(shape, dtype=tdt) for _ in range(3)]
    todo = pairs if pairs is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.heads)]
    for b, h in todo:
        for t, a in zip(out, make_head(cfg, b, h, seed)):
            t[b, h].copy_(torch.from_numpy(a))
    return tuple(out)
