"""Oracle (test infrastructure only): plain CPU statement of the NABLA forward path
and of the gradient of its attention step.

Only ``tests/``, the smoke check and the bench's CPU baseline import this
package.  The library under ``block_sparse_attention_blockmean_amd`` never does.
"""
from .nabla_oracle import (
    fractal_index, reorder, block_mean, pooled_logits, row_softmax, cdf_values, cdf_keep,
    block_tiles, sta_mask, block_mask, kv_lists, mask_from_lists, attention_block,
    masked_attention, forward, block_lse, masked_attention_lse, masked_attention_backward,
    sip_probabilities, sip_mask, weighted_block_attention, ibcs_clusters, ibcs_scores,
    ibcs_block_mask, IBCS_CLUSTERS, IBCS_ITERS, IBCS_TIE_EPS,
)

__all__ = [
    "fractal_index", "reorder", "block_mean", "pooled_logits", "row_softmax", "cdf_values",
    "cdf_keep", "block_tiles", "sta_mask", "block_mask", "kv_lists", "mask_from_lists",
    "attention_block", "masked_attention", "forward", "block_lse", "masked_attention_lse",
    "masked_attention_backward", "sip_probabilities", "sip_mask", "weighted_block_attention",
    "ibcs_clusters", "ibcs_scores", "ibcs_block_mask", "IBCS_CLUSTERS", "IBCS_ITERS", "IBCS_TIE_EPS",
]
