"""Single-GPU emulation of the vocabulary-sharded (tensor-parallel) classifier head.

C is split into row shards, as if each lived on its own device.  The forward runs
cce_forward_shard per shard (LSE over the shard's rows and the target logit where the target
is one of them), stacks the per-shard (lse, target logit) pairs -- on several devices this is
one all-gather of 2 floats per token and shard -- and merges them with cce_merge_shards.  The
backward runs cce_backward_shard per shard with the merged LSE: each shard's rows of dC are
local, and the shards' dE terms are summed, which on several devices is one all-reduce of N x D.
Here the gather is a stack and the all-reduce an add on one GPU; every other step runs in
libcce's kernels.
"""
from __future__ import annotations

import torch

from . import _lib


def shard_bounds(V: int, n_shards: int) -> list[int]:
    """Row boundaries of n_shards near-equal shards, each a multiple of 64 rows except the last,
    so the 64-row filter blocks of each shard line up with those of the full vocabulary."""
    if n_shards < 1 or n_shards > V:
        raise ValueError("need 1 <= n_shards <= V")
    per = -(-V // n_shards)
    per = -(-per // 64) * 64
    b = [min(V, i * per) for i in range(n_shards)] + [V]
    if len(set(b)) != len(b):
        raise ValueError(f"V={V} is too small for {n_shards} shards of whole 64-row blocks")
    return b


def forward_backward(E, C, targets, bounds, ignore_index: int = -100, filter_eps: float = 0.0,
                     dloss=None, grad_dtype=None, err_flag=None):
    """Loss, LSE, dE and dC of sum_n dloss[n] loss[n] (dloss defaults to ones), computed shard
    by shard over the row boundaries `bounds` (0 = b_0 < b_1 < ... < b_S = V)."""
    N, D = E.shape
    V = C.shape[0]
    if bounds[0] != 0 or bounds[-1] != V or any(a >= b for a, b in zip(bounds, bounds[1:])):
        raise ValueError("bounds must rise strictly from 0 to V")
    S = len(bounds) - 1
    dev = E.device
    lse_s = torch.empty((S, N), dtype=torch.float32, device=dev)
    zt_s = torch.empty((S, N), dtype=torch.float32, device=dev)
    tmax_s = []                          # each shard keeps its tile maxima for its backward
    for s in range(S):
        v0, v1 = bounds[s], bounds[s + 1]
        tmax_s.append(_lib.tile_max_buffer(E, C[v0:v1]))
        _lib.cce_forward_shard(E, C[v0:v1], targets, v0, ignore_index, lse=lse_s[s],
                               target_logit=zt_s[s], tile_max=tmax_s[s])
    loss, lse = _lib.cce_merge_shards(lse_s, zt_s, targets, V, ignore_index, err_flag=err_flag)
    if dloss is None:
        dloss = torch.ones(N, dtype=torch.float32, device=dev)
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    dC = torch.empty((V, D), dtype=gdt, device=dev)
    dE = torch.zeros((N, D), dtype=torch.float32, device=dev)
    for s in range(S):
        v0, v1 = bounds[s], bounds[s + 1]
        dE_s, _ = _lib.cce_backward_shard(dloss, E, C[v0:v1], targets, lse, v0, ignore_index,
                                          filter_eps, tile_max=tmax_s[s], dC=dC[v0:v1],
                                          grad_dtype=gdt)
        dE += dE_s                      # the all-reduce over devices
    return loss, lse, dE.to(gdt), dC
