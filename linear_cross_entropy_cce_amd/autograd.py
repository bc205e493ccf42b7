"""torch.autograd integration of libcce: the Cut Cross-Entropy loss as a differentiable op.

    loss = linear_cross_entropy(E, C, targets, ignore_index=-100, filter_eps=2**-12,
                                reduction="mean", entry_floor=0.0)

E [N,D] (token embeddings) and C [V,D] (classifier rows) are CUDA tensors of one dtype (bf16 or
fp32); targets [N] int64.  The loss of token n is lse_v(E_n . C_v) - E_n . C_t(n), 0 for ignored
tokens (the Cut Cross-Entropy abstract, taxoreview.com page dblp:393/3562, sentences 4-6); the
backward skips 64 x 64 blocks of the softmax gradient whose entries are all below filter_eps
(sentence 9; 0 disables it) and, only if entry_floor > 0, drops single non-target entries
whose softmax value is below entry_floor.

Every step of the computation runs in libcce's kernels (cce_forward / cce_backward /
cce_loss_mean, which return the gradients in the dtype of E and C, accumulated in fp32); this
module only routes tensors and gradients:
  * "none" and "sum" keep the forward's tile maxima (when filtering) for the backward, which
    then skips the recompute of tiles they prove negligible;
  * "none": per-token losses; the backward passes the upstream gradient as libcce's dloss;
  * "sum":  the per-token losses summed (dloss = the upstream scalar for every token);
  * "mean": libcce's mean call, which returns the mean over non-ignored tokens together with
    its gradients in one pass; the backward scales them in place by the upstream scalar (so
    it runs once per forward).
"""
from __future__ import annotations

import torch

from . import _lib

FILTER_EPS = 2.0 ** -12


class _PerToken(torch.autograd.Function):
    @staticmethod
    def forward(ctx, E, C, targets, ignore_index, filter_eps, entry_floor):
        tmax = _lib.tile_max_buffer(E, C) if filter_eps > 0 else None
        loss, lse = _lib.cce_forward(E, C, targets, ignore_index, tile_max=tmax)
        ctx.save_for_backward(E, C, targets, lse, tmax)
        ctx.ignore_index = ignore_index
        ctx.filter_eps = filter_eps
        ctx.entry_floor = entry_floor
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        E, C, targets, lse, tmax = ctx.saved_tensors
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1]):
            return None, None, None, None, None, None
        dloss = grad_loss.to(torch.float32).contiguous()
        dE, dC = _lib.cce_backward(dloss, E, C, targets, lse, ctx.ignore_index, ctx.filter_eps,
                                   entry_floor=ctx.entry_floor, tile_max=tmax,
                                   grad_dtype=E.dtype)
        return (dE if ctx.needs_input_grad[0] else None,
                dC if ctx.needs_input_grad[1] else None, None, None, None, None)


class _Sum(torch.autograd.Function):
    @staticmethod
    def forward(ctx, E, C, targets, ignore_index, filter_eps, entry_floor):
        tmax = _lib.tile_max_buffer(E, C) if filter_eps > 0 else None
        loss, lse = _lib.cce_forward(E, C, targets, ignore_index, tile_max=tmax)
        ctx.save_for_backward(E, C, targets, lse, tmax)
        ctx.ignore_index = ignore_index
        ctx.filter_eps = filter_eps
        ctx.entry_floor = entry_floor
        return loss.sum()

    @staticmethod
    def backward(ctx, grad_sum):
        E, C, targets, lse, tmax = ctx.saved_tensors
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1]):
            return None, None, None, None, None, None
        dloss = grad_sum.to(torch.float32).reshape(1).contiguous()   # one scalar for all tokens
        dE, dC = _lib.cce_backward(dloss, E, C, targets, lse, ctx.ignore_index, ctx.filter_eps,
                                   entry_floor=ctx.entry_floor, tile_max=tmax,
                                   grad_dtype=E.dtype)
        return (dE if ctx.needs_input_grad[0] else None,
                dC if ctx.needs_input_grad[1] else None, None, None, None, None)


class _Mean(torch.autograd.Function):
    @staticmethod
    def forward(ctx, E, C, targets, ignore_index, filter_eps, entry_floor):
        mean, n_valid, dE, dC = _lib.cce_loss_mean(E, C, targets, ignore_index, filter_eps,
                                                   entry_floor=entry_floor, grad_dtype=E.dtype)
        ctx.save_for_backward(dE, dC)
        ctx.mark_non_differentiable(n_valid)
        return mean.reshape(()), n_valid.reshape(())

    @staticmethod
    def backward(ctx, grad_mean, _grad_n):
        # The gradients computed by the forward are scaled in place (no second copy of dC),
        # so this backward can run once per forward.
        if getattr(ctx, "used", False):
            raise RuntimeError("linear_cross_entropy(reduction='mean') supports one backward "
                               "per forward; use reduction='sum' or 'none' to differentiate "
                               "the same graph twice")
        ctx.used = True
        dE, dC = ctx.saved_tensors
        g = grad_mean.to(dE.dtype)
        gE = dE.mul_(g) if ctx.needs_input_grad[0] else None
        gC = dC.mul_(g) if ctx.needs_input_grad[1] else None
        return gE, gC, None, None, None, None


def linear_cross_entropy(E: torch.Tensor, C: torch.Tensor, targets: torch.Tensor,
                         ignore_index: int = -100, filter_eps: float = FILTER_EPS,
                         reduction: str = "mean", entry_floor: float = 0.0) -> torch.Tensor:
    """Cross-entropy of the logits E @ C.T against targets, without materialising the logits.

    reduction: "mean" (over non-ignored tokens; 0 when every token is ignored), "sum" or
    "none" (per-token losses, 0 for ignored tokens).  E, C: CUDA, contiguous, same dtype
    (bf16 or fp32); targets: int64 [N].  entry_floor > 0 opts into dropping single
    non-target softmax entries below it in the backward (0: only the block filter)."""
    args = (E, C, targets, int(ignore_index), float(filter_eps), float(entry_floor))
    if reduction == "none":
        return _PerToken.apply(*args)
    if reduction == "sum":
        return _Sum.apply(*args)
    if reduction == "mean":
        mean, _ = _Mean.apply(*args)
        return mean
    raise ValueError(f"reduction must be 'mean', 'sum' or 'none', not {reduction!r}")


class LinearCrossEntropy(torch.nn.Module):
    """Module form of linear_cross_entropy: forward(E, C, targets)."""

    def __init__(self, ignore_index: int = -100, filter_eps: float = FILTER_EPS,
                 reduction: str = "mean", entry_floor: float = 0.0):
        super().__init__()
        if reduction not in ("mean", "sum", "none"):
            raise ValueError(f"reduction must be 'mean', 'sum' or 'none', not {reduction!r}")
        self.ignore_index, self.filter_eps, self.reduction = ignore_index, filter_eps, reduction
        self.entry_floor = entry_floor

    def forward(self, E: torch.Tensor, C: torch.Tensor, targets: torch.Tensor) -> torch.Tensor:
        return linear_cross_entropy(E, C, targets, self.ignore_index, self.filter_eps,
                                    self.reduction, self.entry_floor)

    def extra_repr(self) -> str:
        return (f"ignore_index={self.ignore_index}, filter_eps={self.filter_eps}, "
                f"reduction={self.reduction!r}, entry_floor={self.entry_floor}")
