"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package only draws numbers. It holds none of the method's arithmetic (no
reordering, pooling, softmax, thresholding or attention), so the oracle and the
HIP path can both consume it without sharing any computation.
"""
from .configs import CONFIGS, Config, get_config
from .video_inputs import make_head, make_qkv, GENERATOR_VERSION

__all__ = ["CONFIGS", "Config", "get_config", "make_head", "make_qkv", "GENERATOR_VERSION"]
