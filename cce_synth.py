"""Seeded synthetic inputs for the Cut Cross-Entropy head (shared by tests, bench and smoke).

This module only draws random inputs.  It holds none of the method's arithmetic (no logits,
no log-sum-exp, no gradients), so both the CPU oracle and the GPU path can take their inputs
from it without sharing any of the computation they are compared on.

Workloads.  The abstract of the Cut Cross-Entropy paper (taxoreview.com page dblp:393/3562,
sentences 1-3 and 8) motivates large-vocabulary classifier heads and names Gemma 2 (2B); it gives
no batch, sequence length or data.  The five named workloads below are synthetic stand-ins with
the head shapes of the models they are named after (no weights or hidden states are used):

  tiny            N=256,   D=64,   V=1000,   fp32, uniform targets
  gemma2_2b_head  N=8192,  D=2304, V=256000, bf16, Zipf(1.1) targets, logit std ~3
  llama3_8b_head  N=8192,  D=4096, V=128256, bf16, Zipf(1.1) targets, logit std ~3
  long_seq        N=65536, D=2048, V=32000,  bf16, Zipf(1.0), 20% ignored, logit std ~2
  sparse_stress   N=16384, D=3584, V=256000, bf16, Zipf(1.2), logit std ~8, 5% of rows x2

Recipe (fixed here, the pages are silent):
  * numpy Generator(PCG64) streams; large arrays are drawn in fixed row blocks, each block from
    its own child stream of SeedSequence(seed), so the values do not depend on thread count;
  * E ~ N(0,1); C ~ N(0,1/D) * c_scale; bf16 workloads round both to bf16 (round to nearest
    even) and keep the bf16 values in float32 arrays (exactly representable);
  * targets: Zipf(s) over ids 0..V-1 (P(id) proportional to (id+1)^-s), drawn by inverse CDF,
    or uniform; an optional Bernoulli(p) mask replaces targets by ignore_index;
  * boosted rows (sparse_stress): exactly round(0.05 V) rows of C, chosen without replacement,
    are multiplied by 2 (exact in bf16).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, replace

import numpy as np

IGNORE_INDEX = -100
FILTER_EPS = 2.0 ** -12


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    D: int
    V: int
    dtype: str            # "f32" or "bf16": the type of E and C
    c_scale: float        # C ~ N(0, 1/D) * c_scale
    zipf_s: float | None  # None = uniform targets
    ignore_frac: float = 0.0
    boost_frac: float = 0.0
    boost_factor: float = 2.0
    filter_eps: float = 0.0
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 64, 1000, "f32", 1.0, None, seed=1001),
    "gemma2_2b_head": Workload("gemma2_2b_head", 8192, 2304, 256000, "bf16", 3.0, 1.1,
                               filter_eps=FILTER_EPS, seed=1002),
    "llama3_8b_head": Workload("llama3_8b_head", 8192, 4096, 128256, "bf16", 3.0, 1.1,
                               filter_eps=FILTER_EPS, seed=1003),
    "long_seq": Workload("long_seq", 65536, 2048, 32000, "bf16", 2.0, 1.0, ignore_frac=0.2,
                         filter_eps=FILTER_EPS, seed=1004),
    "sparse_stress": Workload("sparse_stress", 16384, 3584, 256000, "bf16", 8.0, 1.2,
                              boost_frac=0.05, filter_eps=FILTER_EPS, seed=1005),
}

_BLOCK_ROWS = 4096


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); result stays float32."""
    x = np.array(x, dtype=np.float32, copy=True)
    u = x.view(np.uint32)   # finite inputs only: the sum below cannot wrap
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return x


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_matrix(seed: int, tag: int, rows: int, cols: int, std: float, bf16: bool) -> np.ndarray:
    """rows x cols float32 N(0, std^2), drawn in row blocks from child streams of (seed, tag)."""
    out = np.empty((rows, cols), dtype=np.float32)
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS
    children = np.random.SeedSequence([seed, tag]).spawn(max(nblk, 1))

    def fill(b: int) -> None:
        r0, r1 = b * _BLOCK_ROWS, min(rows, (b + 1) * _BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(children[b]))
        blk = out[r0:r1]
        g.standard_normal(out=blk, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if bf16:
            u = blk.view(np.uint32)
            u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
            u &= np.uint32(0xFFFF0000)

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """n iid ids in [0, V) with P(id) proportional to (id + 1)^-s (inverse-CDF sampling)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)


def make_inputs(w: Workload, N: int | None = None) -> dict:
    """E [N,D], C [V,D] (float32 arrays; bf16-exact for bf16 workloads) and targets [N] int64.

    N overrides the token count (the first N rows of the full draw are identical for any N,
    since rows come in fixed blocks)."""
    N = w.N if N is None else N
    bf = w.dtype == "bf16"
    E = normal_matrix(w.seed, 1, N, w.D, 1.0, bf)
    C = normal_matrix(w.seed, 2, w.V, w.D, w.c_scale / np.sqrt(w.D), bf)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 3])))
    if w.boost_frac > 0:
        k = int(round(w.boost_frac * w.V))
        rows = rng.choice(w.V, size=k, replace=False)
        C[rows] *= np.float32(w.boost_factor)   # a power of two: stays bf16-exact
    else:
        rows = np.zeros(0, dtype=np.int64)
    if w.zipf_s is None:
        t = rng.integers(0, w.V, size=N, dtype=np.int64)
    else:
        t = zipf_targets(rng, N, w.V, w.zipf_s)
    if w.ignore_frac > 0:
        mask = rng.random(N) < w.ignore_frac
        t[mask] = IGNORE_INDEX
    return {"E": E, "C": C, "targets": t, "boosted_rows": np.sort(rows)}


def small_case(N: int, D: int, V: int, dtype: str = "bf16", seed: int = 0, c_scale: float = 3.0,
               zipf_s: float | None = 1.1, ignore_frac: float = 0.0) -> dict:
    """A small custom case drawn with the same recipe (for parity tests spanning a few tiles)."""
    w = Workload(f"case{N}x{D}x{V}", N, D, V, dtype, c_scale, zipf_s, ignore_frac=ignore_frac,
                 seed=seed)
    return make_inputs(w)


def dloss_weights(seed: int, N: int) -> np.ndarray:
    """Per-token upstream gradients ~ U(0.5, 1.5) as float32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
    return (0.5 + g.random(N)).astype(np.float32)
