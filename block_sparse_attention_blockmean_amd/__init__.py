"""NABLA block-mean adaptive block-sparse attention for MI355X (gfx950): the forward
path and the gradient of its attention step.

Python face of libnabla.so: ``reorder``, ``build_mask``, ``attn_fwd``, ``attn_bwd`` take torch
device tensors, pass their pointers and the current HIP stream to the C ABI in
``include/nabla.h``, and raise on any error.  Build the library with
``python -m block_sparse_attention_blockmean_amd.build``.
"""
from ._binding import (
    EXPORTS, LIB_PATH, NablaError, StaWindow, attn_bwd, attn_bwd_workspace_size, attn_fwd,
    attn_fwd_raster, attn_fwd_weighted, build_mask, build_mask_raster_noalloc, build_mask_sip,
    build_mask_workspace_size,
    load_library, reorder,
)

__all__ = [
    "EXPORTS", "LIB_PATH", "NablaError", "StaWindow", "attn_bwd", "attn_bwd_workspace_size",
    "attn_fwd", "attn_fwd_raster", "attn_fwd_weighted", "build_mask", "build_mask_raster_noalloc",
    "build_mask_sip",
    "build_mask_workspace_size", "load_library", "reorder",
]
