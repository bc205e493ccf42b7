"""The Python binding refuses malformed arguments before anything reaches the library: wrong
dtype, shape, device or layout of an input, output, workspace or flag array."""
import pytest
import torch

import linear_cross_entropy_cce_amd as cce
from gpu_helpers import DEV, II

pytestmark = pytest.mark.gpu

N, D, V = 100, 64, 300


def _case():
    g = torch.Generator().manual_seed(7)
    E = torch.randn(N, D, generator=g).to(DEV, torch.bfloat16)
    C = torch.randn(V, D, generator=g).to(DEV, torch.bfloat16)
    t = torch.randint(0, V, (N,), generator=g).to(DEV)
    return E, C, t


def test_forward_arguments_are_checked():
    E, C, t = _case()
    with pytest.raises(ValueError):
        cce.cce_forward(E.cpu(), C, t, II)                       # input on the host
    with pytest.raises(ValueError):
        cce.cce_forward(E.t(), C, t, II)                         # not contiguous (and [D,N])
    with pytest.raises(TypeError):
        cce.cce_forward(E, C.float(), t, II)                     # mixed dtypes
    with pytest.raises(ValueError):
        cce.cce_forward(E, C, t.int(), II)                       # int32 targets
    with pytest.raises(ValueError):
        cce.cce_forward(E, C, t, II, loss=torch.empty(N + 1, device=DEV))
    with pytest.raises(ValueError):
        cce.cce_forward(E, C, t, II, ws=torch.empty(1 << 20, dtype=torch.uint8))   # host ws
    with pytest.raises(ValueError):
        cce.cce_forward(E, C, t, II, err_flag=torch.zeros(1, dtype=torch.int64, device=DEV))
    with pytest.raises(cce.CCEError):
        cce.cce_forward(E, C, t, II, ws=torch.empty(8, dtype=torch.uint8, device=DEV))
    loss, lse = cce.cce_forward(E, C, t, II)                     # the well-formed call works
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all() and torch.isfinite(lse).all()


def test_backward_arguments_are_checked():
    E, C, t = _case()
    loss, lse = cce.cce_forward(E, C, t, II)
    dl = torch.ones(N, device=DEV)
    with pytest.raises(ValueError):
        cce.cce_backward(dl.cpu(), E, C, t, lse, II)            # dloss on the host
    with pytest.raises(ValueError):
        cce.cce_backward(dl.double(), E, C, t, lse, II)         # float64 dloss
    with pytest.raises(ValueError):
        cce.cce_backward(torch.ones(N - 1, device=DEV), E, C, t, lse, II)
    with pytest.raises(ValueError):
        cce.cce_backward(dl, E, C, t, lse, II, dE=torch.empty(N, D, device=DEV),
                         grad_dtype=torch.bfloat16)              # dE not in grad_dtype
    with pytest.raises(ValueError):
        cce.cce_backward(dl, E, C, t, lse, II, dC=torch.empty(V, D + 8, device=DEV))
    with pytest.raises(ValueError):
        cce.cce_backward(dl, E, C, t, lse, II,
                         skip_stats=torch.zeros(2, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        cce.cce_backward(dl, E, C, t, lse, II, tile_max=torch.empty(3, device=DEV))
    with pytest.raises(cce.CCEError):
        cce.cce_backward(dl, E, C, t, lse, II, -1.0)             # negative threshold
    with pytest.raises(cce.CCEError):
        cce.cce_backward(dl, E, C, t, lse, II, 0.0, entry_floor=float("nan"))
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, 2.0 ** -12)
    torch.cuda.synchronize()
    assert torch.isfinite(dE).all() and torch.isfinite(dC).all()
