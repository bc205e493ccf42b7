#!/usr/bin/env python3
"""Benchmark of the Cut Cross-Entropy hot path (libcce) on one MI355X.

One step = cce_forward (per-token loss and LSE) + cce_backward (dE, dC with gradient
filtering) over one batch of synthetic input already resident in device memory.  The default
workload is the Gemma-2-2B-shaped head (N=8192 tokens, D=2304, V=256000, bf16, Zipf(1.1)
targets, filter_eps=2^-12).  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Flop accounting.  The method's work (pct_bf16_peak, roofline): 2 N V D for the forward; for
the backward 2 N V D for the logit recompute, less the 256 x 256 tiles that the forward's
tile maxima prove negligible (never recomputed), plus 4 N V D for the dE and dC products,
less the 64 x 64 blocks of G that the filter skips.  With nothing filtered this is the
8 N V D of the dense computation, which is also reported, labelled as dense-equivalent.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix), published
HBM_PEAK_GBS = 8000.0
SOURCES = ("linear_cross_entropy_cce_amd/csrc/cce_api.hip",
           "linear_cross_entropy_cce_amd/csrc/cce_kernels.hpp",
           "linear_cross_entropy_cce_amd/csrc/tile_engine.hpp")


def kernel_source_hash() -> str:
    """Hash of the sources of the kernels and their launch plan (the profiles record it)."""
    h = hashlib.sha256()
    for p in SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def tiles_proved_negligible(tmax, lse, t, N: int, V: int, eps: float) -> int:
    """256 x 256 (token, vocabulary) tiles whose recompute the backward skips: the largest
    logit of the tile (the forward's tile maxima, in log2 units) less the smallest LSE of the
    tile's non-ignored tokens lies below log2(eps) by the kernel's margin of 2^-10, and no token
    of the tile has its target among the tile's rows.  Counted on the GPU after the timed
    region, for the flop accounting."""
    import math
    import torch
    if eps <= 0:
        return 0
    n_tb, n_vt = -(-N // 256), -(-V // 256)
    tm = tmax[:n_tb * n_vt * 8].view(n_tb, n_vt, 8).amax(dim=2)
    l2 = lse * (1.0 / math.log(2.0))
    valid = t != -100
    pad = n_tb * 256 - N
    l2v = torch.where(valid, l2, torch.full_like(l2, float("inf")))
    lmin = torch.nn.functional.pad(l2v, (0, pad), value=float("inf")).view(n_tb, 256).amin(dim=1)
    below = (tm - lmin[:, None]) < (math.log2(eps) - 2.0 ** -10)
    has_t = torch.zeros(n_tb, n_vt, dtype=torch.bool, device=t.device)
    tok = torch.arange(N, device=t.device)
    has_t[tok[valid] // 256, t[valid] // 256] = True
    return int((below & ~has_t).sum())


def cpu_baseline(d, w, n_tokens: int) -> dict:
    """The CPU oracle as it stands, on the first n_tokens (whole 64-token blocks) of the same
    workload: their loss, LSE, dE rows and their contribution to dC over the full vocabulary."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max([i.get("num_threads", 1) for i in pools] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools}))
    except Exception:  # pragma: no cover
        cores, blas = os.cpu_count() or 1, "unknown"
    rows = np.arange(n_tokens)
    t0 = time.perf_counter()
    oracle.token_rows(d["E"], d["C"], d["targets"], rows, np.full(n_tokens, 1.0 / w.N),
                      -100, filter_eps=w.filter_eps)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tokens} tokens of {w.name} (float64 forward, backward and dC "
                      f"contribution over all V={w.V}), {dt:.1f} s", "blas": blas}


def vendor_gemm_reference(dev) -> dict:
    """Context for the MFMA roofline: the vendor library GEMM (torch.mm, hipBLASLt on ROCm) on
    random bf16 operands of the forward's shape class, timed on the same GPU in the same run.
    Dense bf16 MFMA throughput with random data is bounded by the board's power limit well
    below the published peak; this number shows where that bound sits right now."""
    import torch
    M, Nn, K = 8192, 32768, 2304
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(K, Nn, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(M, Nn, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 20
    s.record()
    for _ in range(iters):
        torch.mm(a, b, out=c)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    return {"op": f"torch.mm bf16 randn {M}x{K} @ {K}x{Nn}", "tflops": 2.0 * M * Nn * K / (ms * 1e-3) / 1e12}


def sample_clock(step, seconds: float = 2.5) -> dict | None:
    """GFX clock and board power while the step runs back to back (outside the timed region):
    amd-smi is polled from a thread; its readings refresh about once a second."""
    import re
    import shutil
    import subprocess
    import threading
    import torch
    if shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True,
                                   text=True, timeout=10).stdout
            except Exception:  # pragma: no cover
                return
            p = re.search(r"SOCKET_POWER:\s*(\d+)", r)
            clk = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)", r)]
            if p and clk:
                samples.append((float(p.group(1)), sum(clk) / len(clk)))
            stop.wait(0.2)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    busy = samples[1:] if len(samples) > 2 else samples   # first reading may predate the load
    if not busy:
        return None
    mhz = sum(c for _, c in busy) / len(busy)
    return {"gfx_mhz_mean": mhz, "socket_power_w_mean": sum(p for p, _ in busy) / len(busy),
            "samples": len(busy), "how": f"amd-smi polled while the step ran {seconds} s back to back",
            "bf16_dense_peak_at_this_clock_tflops": 256 * 4096 * mhz * 1e6 / 1e12}


def copy_calibration() -> int:
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
    return 0


def memory_compare(workload: str) -> int:
    """Peak device memory and time of one forward + backward of the classifier-head loss at the
    workload's shape: a plain PyTorch head (logits materialised by a library GEMM, then
    log-softmax, NLL and autograd's backward) against libcce through its autograd wrapper.
    Prints one JSON line.  Context for the pages' Gemma 2 (2B) memory figures, not a parity
    check (their N and hardware are not given)."""
    import torch
    import torch.nn.functional as F

    import cce_synth as S
    from linear_cross_entropy_cce_amd import linear_cross_entropy
    w = S.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = S.make_inputs(w)
    E0 = torch.from_numpy(d["E"]).to(dev, tdt)
    C0 = torch.from_numpy(d["C"]).to(dev, tdt)
    t = torch.from_numpy(d["targets"]).to(dev)

    def naive(E, C):
        logits = F.linear(E, C).float()
        return F.cross_entropy(logits, t, ignore_index=S.IGNORE_INDEX)

    def cce_head(E, C):
        return linear_cross_entropy(E, C, t, S.IGNORE_INDEX, w.filter_eps, "mean")

    out = {"workload": f"{w.name}: N={w.N} D={w.D} V={w.V} {w.dtype}"}
    for name, fn in (("pytorch_materialised", naive), ("libcce", cce_head)):
        E = E0.detach().clone().requires_grad_(True)
        C = C0.detach().clone().requires_grad_(True)
        fn(E, C).backward()                      # warm-up (allocator, libraries)
        E.grad = C.grad = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        t0 = time.perf_counter()
        loss = fn(E, C)
        loss.backward()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        peak = torch.cuda.max_memory_allocated() - base
        grads = E.grad.numel() * E.grad.element_size() + C.grad.numel() * C.grad.element_size()
        out[name] = {"loss": float(loss.item()), "ms": ms, "peak_bytes_above_inputs": int(peak),
                     "gradient_bytes": int(grads),
                     "peak_minus_gradients": int(peak - grads)}
        del E, C, loss
    out["ratio_peak_minus_gradients"] = (out["pytorch_materialised"]["peak_minus_gradients"] /
                                         max(out["libcce"]["peak_minus_gradients"], 1))
    print(json.dumps(out), flush=True)
    return 0


def shards_compare(workload: str, n_shards: int, steps: int, warmup: int) -> int:
    """The vocabulary-sharded head emulated on one GPU (one JSON line): a fwd+bwd step through
    S shards of C (cce_forward_shard per shard, cce_merge_shards, cce_backward_shard per shard
    with the merged LSE, dE terms summed) against the unsharded step, and the per-shard kernel
    times, i.e. the work of one device of an S-way tensor-parallel head at its real shape."""
    import torch

    import cce_synth as S
    import linear_cross_entropy_cce_amd as cce
    from linear_cross_entropy_cce_amd import sharded
    w = S.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = S.make_inputs(w)
    E = torch.from_numpy(d["E"]).to(dev, tdt)
    C = torch.from_numpy(d["C"]).to(dev, tdt)
    t = torch.from_numpy(d["targets"]).to(dev)
    dl = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=dev)
    bounds = sharded.shard_bounds(w.V, n_shards)

    def sharded_step():
        return sharded.forward_backward(E, C, t, bounds, S.IGNORE_INDEX, w.filter_eps, dloss=dl)

    tmax = cce.tile_max_buffer(E, C)

    def plain_step():
        loss, lse = cce.cce_forward(E, C, t, S.IGNORE_INDEX, tile_max=tmax)
        return cce.cce_backward(dl, E, C, t, lse, S.IGNORE_INDEX, w.filter_eps, tile_max=tmax)

    out = {"workload": f"{w.name}: N={w.N} D={w.D} V={w.V} {w.dtype}", "shards": n_shards,
           "shard_rows": [b - a for a, b in zip(bounds, bounds[1:])]}
    for name, fn in (("unsharded", plain_step), ("sharded", sharded_step)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        cce.timing_begin(max_launches=steps * (60 * n_shards + 200))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        k = cce.timing_end()
        out[name] = {"ms_per_step": a.elapsed_time(b) / steps,
                     "kernel_ms_per_step": {kk: v[0] / steps for kk, v in k.items()}}
    sh = out["sharded"]["kernel_ms_per_step"]
    out["per_shard_ms"] = {"forward": (sh.get("fwd_lse", 0.0) + sh.get("fwd_finish", 0.0)) / n_shards,
                           "backward": (sh.get("bwd_g", 0.0) + sh.get("bwd_fused", 0.0)) / n_shards}
    print(json.dumps(out), flush=True)
    return 0


def vocab_order_compare(workload: str, steps: int, warmup: int) -> int:
    """A fwd+bwd step on the workload as given and on the same problem with the vocabulary
    relabelled (one JSON line): the classifier rows sorted by decreasing L2 norm and the targets
    mapped accordingly, which gathers the rows that carry most of the softmax into few
    vocabulary tiles, so whole K stages of the gradient products are skipped.  The relabelling
    is the caller's (done here with torch, outside the timed region; a training loop would keep
    its classifier in that order); the loss and dE are unchanged and dC comes back in the new
    row order.  The results of the two runs are compared, untimed."""
    import torch

    import cce_synth as S
    import linear_cross_entropy_cce_amd as cce
    w = S.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = S.make_inputs(w)
    E = torch.from_numpy(d["E"]).to(dev, tdt)
    C = torch.from_numpy(d["C"]).to(dev, tdt)
    t = torch.from_numpy(d["targets"]).to(dev)
    dl = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    perm = torch.argsort(torch.linalg.vector_norm(C.float(), dim=1), descending=True)
    rank = torch.empty_like(perm)
    rank[perm] = torch.arange(w.V, device=dev)
    Cp = C[perm].contiguous()
    tp = torch.where(t == S.IGNORE_INDEX, t, rank[t.clamp(min=0)])
    b.record()
    torch.cuda.synchronize()
    out = {"workload": f"{w.name}: N={w.N} D={w.D} V={w.V} {w.dtype}, filter_eps={w.filter_eps:g}",
           "order": "classifier rows by decreasing L2 norm",
           "relabel_ms_untimed": a.elapsed_time(b)}
    res = {}
    for name, CC, tt in (("as_given", C, t), ("relabelled", Cp, tp)):
        stats = torch.zeros(2, dtype=torch.int64, device=dev)
        tmax = cce.tile_max_buffer(E, CC)

        def step():
            loss, lse = cce.cce_forward(E, CC, tt, S.IGNORE_INDEX, tile_max=tmax)
            dE, dC = cce.cce_backward(dl, E, CC, tt, lse, S.IGNORE_INDEX, w.filter_eps,
                                      tile_max=tmax, skip_stats=stats)
            return loss, dE, dC
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        cce.timing_begin(max_launches=steps * 200)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        k = cce.timing_end()
        skipped, total = (int(x) for x in stats.tolist())
        out[name] = {"ms_per_step": a.elapsed_time(b) / steps,
                     "kernel_ms_per_step": {kk: v[0] / steps for kk, v in k.items()},
                     "skip_fraction_64x64_blocks": skipped / total if total else 0.0}
        res[name] = step()
    (l0, e0, c0), (l1, e1, c1) = res["as_given"], res["relabelled"]
    torch.cuda.synchronize()
    rel = lambda x, y: float((x - y).norm() / y.norm().clamp(min=1e-30))
    out["relabelled_vs_as_given"] = {"loss_max_abs": float((l1 - l0).abs().max()),
                                     "dE_rel": rel(e1, e0), "dC_rel": rel(c1, c0[perm])}
    out["speedup"] = out["as_given"]["ms_per_step"] / out["relabelled"]["ms_per_step"]
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gemma2_2b_head")
    ap.add_argument("--filter-eps", type=float, default=None,
                    help="override the workload's gradient filter threshold")
    ap.add_argument("--entry-floor", type=float, default=0.0,
                    help="optional entry floor of the backward (0: off, the block filter only)")
    ap.add_argument("--no-tile-max", action="store_true",
                    help="do not pass the forward's tile maxima to the backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--shards", type=int, default=0,
                    help="only time the vocabulary-sharded head emulated on one GPU with this "
                         "many shards against the unsharded step (one JSON line)")
    ap.add_argument("--memory-compare", action="store_true",
                    help="only compare peak device memory of a materialising PyTorch head with "
                         "libcce at the workload's shape (one JSON line)")
    ap.add_argument("--vocab-order", action="store_true",
                    help="only time the workload with its vocabulary relabelled by classifier "
                         "row norm against the workload as given (one JSON line)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the GPU clock / power sampling after the timed region")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the vendor-GEMM reference measurement (context only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times): the reference kernel "
                         "for scaling the HBM byte counters of a profiler")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.memory_compare:
        return memory_compare(args.workload)
    if args.shards:
        return shards_compare(args.workload, args.shards, args.steps, args.warmup)
    if args.vocab_order:
        return vocab_order_compare(args.workload, args.steps, args.warmup)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: libcce is measured on one GPU only (asked for {max(args.gpus, world)}); "
              "sharding the head over several GPUs is described, not benchmarked.",
              file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import cce_synth as S
    import linear_cross_entropy_cce_amd as cce

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = S.WORKLOADS[args.workload]
    eps = w.filter_eps if args.filter_eps is None else args.filter_eps
    N, V, D = w.N, w.V, w.D
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    d = S.make_inputs(w)
    gen_s = time.perf_counter() - t0
    E = torch.from_numpy(d["E"]).to(dev, tdt)
    C = torch.from_numpy(d["C"]).to(dev, tdt)
    t = torch.from_numpy(d["targets"]).to(dev)
    dloss = torch.full((N,), 1.0 / N, dtype=torch.float32, device=dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    dE = torch.empty((N, D), dtype=torch.float32, device=dev)
    dC = torch.empty((V, D), dtype=torch.float32, device=dev)
    stats = torch.zeros(2, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    fws_b = cce.forward_workspace_bytes(N, V, D, tdt)
    bws_b = cce.backward_workspace_bytes(N, V, D, tdt, torch.float32)
    fws = cce._lib.workspace(fws_b, dev)
    bws = cce._lib.workspace(bws_b, dev)
    # the forward's tile maxima, kept for the backward (N x V / 2048 bytes)
    tmax = None if args.no_tile_max else cce.tile_max_buffer(E, C)
    tmax_b = 0 if tmax is None else tmax.numel() * 4
    torch.cuda.reset_peak_memory_stats()

    def step():
        cce.cce_forward(E, C, t, S.IGNORE_INDEX, loss=loss, lse=lse, tile_max=tmax, ws=fws)
        cce.cce_backward(dloss, E, C, t, lse, S.IGNORE_INDEX, eps, entry_floor=args.entry_floor,
                         tile_max=tmax, dE=dE, dC=dC, ws=bws, skip_stats=stats)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base_alloc

    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    cce.timing_begin(max_launches=args.steps * 200)
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    kernels = cce.timing_end()
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    clock = None if args.no_clock else sample_clock(step)

    skipped, total_blocks = (int(x) for x in stats.tolist())
    n_valid = int((d["targets"] != S.IGNORE_INDEX).sum())
    skip_frac = skipped / total_blocks if total_blocks else 0.0
    n_tiles = -(-N // 256) * -(-V // 256)
    tiles_skipped = 0 if tmax is None else tiles_proved_negligible(tmax, lse, t, N, V, eps)
    tile_frac = tiles_skipped / n_tiles
    flop_fwd = 2.0 * N * V * D
    flop_recompute = 2.0 * N * V * D * (1.0 - tile_frac)
    flop_products = 4.0 * N * V * D * (1.0 - skip_frac)
    flop_method = flop_fwd + flop_recompute + flop_products
    tflops = flop_method / (ms * 1e-3) / 1e12
    tflops_dense = 8.0 * N * V * D / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # dominant kernel: the kind with the largest time per step
    per_step = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
                for k, v in kernels.items()}
    # the first pair's recompute runs in bwd_g, the rest in the fused launches.  Blocks and
    # chunks are balanced splits of 256-wide tiles (parts = ceil(tiles / widest part)), the
    # first part floor(tiles / parts) tiles long.
    def first_part(n, widest):
        tiles = -(-n // 256)
        parts = -(-tiles // (widest // 256))
        return min(n, (tiles // parts) * 256)
    nc0 = first_part(N, cce.backward_token_block(N, V, D, tdt))
    vc0 = first_part(V, cce.backward_chunk(N, V, D, tdt))
    first = (nc0 * vc0) / (N * V)
    flops_per_step = {"fwd_lse": flop_fwd,
                      "bwd_g": flop_recompute * first,
                      "bwd_fused": flop_products + flop_recompute * (1.0 - first)}
    dom = max((k for k in per_step if k in flops_per_step), key=lambda k: per_step[k]["ms_per_step"])
    dom_ms_launch = kernels[dom][0] / kernels[dom][1]
    dom_flop_launch = flops_per_step[dom] / per_step[dom]["launches_per_step"]
    achieved = dom_flop_launch / (dom_ms_launch * 1e-3) / 1e12
    for k, v in per_step.items():
        if k in flops_per_step:
            v["tflops"] = flops_per_step[k] / (v["ms_per_step"] * 1e-3) / 1e12
    traffic = traffic_from_profiles(dom, w.name)

    out = {
        "metric": "CCE fwd+bwd tokens/s; TFLOP/s as % bf16 MFMA peak; extra HBM bytes",
        "value": N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": step_ms[len(step_ms) // 2],
        "ms_per_step_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, cce_synth recipe; no model weights)",
        "config": {"workload": f"{w.name}: N={N} D={D} V={V} {w.dtype}, "
                               f"filter_eps={eps:g}", "N": N, "D": D, "V": V,
                   "filter_eps": eps, "entry_floor": args.entry_floor,
                   "tile_max": tmax is not None, "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / peak,
        "flops_counted": "method's work: forward 2NVD, recompute 2NVD less tiles proved "
                         "negligible, dE and dC products 4NVD less skipped 64x64 blocks",
        "tflops_dense_equivalent": tflops_dense,
        "pct_bf16_peak_dense_equivalent": 100.0 * tflops_dense / peak,
        "skip_fraction_64x64_blocks": skip_frac,
        "recompute_tiles_skipped": tiles_skipped,
        "recompute_tiles_total": n_tiles,
        # tokens/s counts every token (ignored ones still cost forward work, since their LSE is
        # returned); the same over non-ignored tokens only:
        "n_valid_tokens": n_valid,
        "tokens_per_s_valid": n_valid / (ms * 1e-3),
        "kernels": per_step,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic},
        "extra_hbm_bytes": {"forward_workspace": fws_b, "backward_workspace": bws_b,
                            "tile_max": tmax_b,
                            "total": fws_b + bws_b + tmax_b,
                            "per_token": (fws_b + bws_b + tmax_b) / N,
                            "allocator_peak_delta": int(peak_extra),
                            "logits_fp32_avoided": 4 * N * V},
        "context": {"pages_gemma2_2b": "loss memory 24 GB -> 1 MB, classifier head 28 GB -> "
                                        "1 GB (hardware not given)"},
        "input_generation_s": gen_s,
        "kernel_source_hash": kernel_source_hash(),
    }
    if clock is not None:
        out["context"]["clock_during_run"] = clock
    if not args.no_gemm_ref:
        out["context"]["vendor_gemm_same_gpu"] = vendor_gemm_reference(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, w, args.cpu_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
