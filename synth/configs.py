"""The five video-shaped attention workloads.

Shapes follow the latent grids of the video models the NABLA summary evaluates
(Wan 2.1, 720p; page "NABLA - Atenção de Bloco Adaptativa de Vizinhança",
section Resultados Experimentais) and the 720p HunyuanVideo / Wan2.1 frame counts
of the AB-Attention news page (section "Como foi a avaliação").  Every tensor is
synthetic; no model weights or prompts are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    B: int
    heads: int
    d: int
    dtype: str            # "f32" or "bf16"
    T: int
    H: int
    W: int
    P: int
    N: int
    thr: float
    sta: Optional[Tuple[int, int, int]] = None   # window in tiles (t, h, w), odd
    thr_list: Tuple[float, ...] = field(default_factory=tuple)  # extra thresholds reported
    scale_logits: bool = True                    # scale Q,K so diagonal logits average 8

    @property
    def L(self) -> int:
        return self.T * self.H * self.W

    @property
    def nb(self) -> int:
        return self.L // self.N

    @property
    def BH(self) -> int:
        return self.B * self.heads

    def tensor_bytes(self) -> int:
        return self.BH * self.L * self.d * (2 if self.dtype == "bf16" else 4)


CONFIGS = [
    Config("tiny", 0, B=1, heads=2, d=64, dtype="f32", T=4, H=16, W=16, P=8, N=64, thr=0.1,
           scale_logits=False),
    Config("wan1.3b_480p", 1, B=1, heads=12, d=128, dtype="bf16", T=21, H=32, W=48, P=8, N=64,
           thr=0.2),
    Config("wan1.3b_480p_sta", 2, B=1, heads=12, d=128, dtype="bf16", T=21, H=32, W=48, P=8, N=64,
           thr=0.2, sta=(3, 3, 3), thr_list=(0.05, 0.2)),
    Config("hunyuan_720p_sta", 3, B=1, heads=24, d=128, dtype="bf16", T=33, H=48, W=80, P=8, N=64,
           thr=0.2, sta=(3, 3, 3)),
    Config("wan14b_720p_cfg", 4, B=2, heads=40, d=128, dtype="bf16", T=21, H=48, W=80, P=8, N=64,
           thr=0.1),
]


def get_config(key) -> Config:
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(key)
