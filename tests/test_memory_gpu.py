"""Device memory of a forward + backward (the Cut Cross-Entropy abstract, sentences 6 and 8:
the loss's extra memory is small): the allocator's peak above the inputs, less the outputs the
caller asked for (loss, LSE, dE, dC) and the upstream gradient, is the workspace the library's
queries report (at most their sum plus 1 MiB), and it grows with the token count by a
per-token slope that does not depend on the vocabulary size (no N x V term)."""
import pytest
import torch

import linear_cross_entropy_cce_amd as cce
from gpu_helpers import DEV, EPS, II, log

pytestmark = pytest.mark.gpu

MIB = 1 << 20


def extra_bytes(N, V, D):
    """Allocator peak of a forward + backward above the inputs, less the outputs and dloss;
    the two workspace queries."""
    g = torch.Generator(device=DEV)
    g.manual_seed(N + V)
    E = torch.randn(N, D, device=DEV, generator=g).to(torch.bfloat16)
    C = (torch.randn(V, D, device=DEV, generator=g) * (3.0 / D ** 0.5)).to(torch.bfloat16)
    t = torch.randint(0, V, (N,), device=DEV, generator=g)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    dl = torch.ones(N, device=DEV)
    loss, lse = cce.cce_forward(E, C, t, II)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, EPS)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    outputs = sum(x.numel() * x.element_size() for x in (dl, loss, lse, dE, dC))
    ws_f = cce.forward_workspace_bytes(N, V, D, torch.bfloat16)
    ws_b = cce.backward_workspace_bytes(N, V, D, torch.bfloat16, torch.float32)
    del E, C, t, dl, loss, lse, dE, dC
    return peak - outputs, ws_f, ws_b


def test_allocator_peak_is_the_workspace():
    """At N = 4096, 8192 and 16384 the peak is at most the two workspace queries plus 1 MiB, and
    at least the backward's (the forward's workspace is released before the backward's is
    taken) less the caching allocator's rounding (ALLOC_SLACK); the queries' per-token slope is
    exactly the same at V = 32000 and V = 256000, and so, up to that rounding over 12288
    tokens, is the measured one."""
    D = 2304
    ALLOC_SLACK = 2 * MIB
    n_lo, n_hi = 4096, 16384
    slope, q_slope = {}, {}
    for V in (32000, 256000):
        got, q = {}, {}
        for N in (n_lo, 8192, n_hi):
            extra, ws_f, ws_b = extra_bytes(N, V, D)
            log(f"[memory] N={N} V={V}: peak beyond inputs and outputs {extra / MIB:.2f} MiB, "
                f"workspace queries {ws_f / MIB:.2f} + {ws_b / MIB:.2f} MiB")
            assert ws_b - ALLOC_SLACK <= extra <= ws_f + ws_b + MIB
            got[N], q[N] = extra, ws_b
        slope[V] = (got[n_hi] - got[n_lo]) / (n_hi - n_lo)
        q_slope[V] = (q[n_hi] - q[n_lo]) / (n_hi - n_lo)
        log(f"[memory] V={V}: {slope[V]:.0f} extra bytes per token (query {q_slope[V]:.0f})")
    # the per-token slope is that of the G store of two pairs (2 x Vc columns of bf16 per
    # token plus flags): exactly the same in the queries, within the rounding when measured
    assert q_slope[32000] == q_slope[256000]
    assert q_slope[256000] <= 2 * 8192 * 2 + 2 * 8192 // 64 / 64 + 1
    assert abs(slope[32000] - slope[256000]) <= 2 * ALLOC_SLACK / (n_hi - n_lo)
