"""Device memory of a forward + backward (SURVEY f3 reading of the Cut Cross-Entropy abstract,
sentences 6 and 8: the loss's extra memory is small): the allocator's peak above the inputs,
less the outputs the caller asked for (loss, LSE, dE, dC) and the upstream gradient, is the
workspace the library's queries report, within 1 MiB, and it grows with the token count by a
per-token slope that does not depend on the vocabulary size (no N x V term)."""
import pytest
import torch

import linear_cross_entropy_cce_amd as cce
from gpu_helpers import DEV, EPS, II, log

pytestmark = pytest.mark.gpu

MIB = 1 << 20


def extra_bytes(N, V, D):
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
    ws = (cce.forward_workspace_bytes(N, V, D, torch.bfloat16)
          + cce.backward_workspace_bytes(N, V, D, torch.bfloat16, torch.float32))
    del E, C, t, dl, loss, lse, dE, dC
    return peak - outputs, ws


def test_allocator_peak_is_the_workspace():
    D = 2304
    slope = {}
    for V in (32000, 256000):
        got = {}
        for N in (4096, 8192):
            extra, ws = extra_bytes(N, V, D)
            log(f"[memory] N={N} V={V}: peak beyond inputs and outputs {extra / MIB:.2f} MiB, "
                f"workspace query {ws / MIB:.2f} MiB")
            assert extra <= ws + MIB
            got[N] = extra
        slope[V] = (got[8192] - got[4096]) / 4096
        log(f"[memory] V={V}: {slope[V]:.0f} extra bytes per token")
    # the per-token slope is that of the G store of two pairs (2 x Vc columns of bf16 per
    # token plus flags), the same at V = 32000 and V = 256000
    assert abs(slope[32000] - slope[256000]) <= 64
    assert slope[256000] <= 2 * 8192 * 2 + 8192 // 64 * 2 / 64 + 64
