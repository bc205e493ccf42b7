"""Cut Cross-Entropy for AMD MI355X (gfx950): Python binding of libcce.

The classifier-head cross-entropy loss, lse_v(E C_v^T) - E C_target^T, and its gradients dE and
dC, computed by hand-written HIP kernels without writing the N x V logits to device memory
(the Cut Cross-Entropy abstract, taxoreview.com page dblp:393/3562, sentences 4-6 and 9).
"""
from ._lib import (KERNEL_KINDS, LIB_PATH, CCEError, backward_chunk, backward_token_block,
                   backward_workspace_bytes, cce_backward, cce_backward_shard, cce_forward,
                   cce_forward_no_workspace, cce_forward_shard, cce_loss_mean, cce_merge_shards,
                   forward_no_workspace_max_bytes, forward_splits, forward_workspace_bytes, lib,
                   loss_mean_workspace_bytes, tile_max_buffer, tile_max_count, timing_begin,
                   timing_end, workspace)
from .autograd import LinearCrossEntropy, linear_cross_entropy

__all__ = ["LinearCrossEntropy", "linear_cross_entropy", "CCEError", "LIB_PATH", "KERNEL_KINDS",
           "backward_chunk", "backward_token_block", "backward_workspace_bytes", "cce_backward",
           "cce_backward_shard", "cce_forward", "cce_forward_no_workspace", "cce_forward_shard",
           "cce_loss_mean", "cce_merge_shards", "forward_no_workspace_max_bytes",
           "forward_splits", "forward_workspace_bytes", "lib", "loss_mean_workspace_bytes",
           "tile_max_buffer", "tile_max_count", "timing_begin", "timing_end", "workspace"]
