"""cce_forward_no_workspace, the forward for callers that cannot allocate, through the C ABI:
its loss, LSE and tile maxima are bitwise those of cce_forward with a caller workspace (same
kernels, same launch plan), on two calls in a row, the second with a smaller input, so the
second call runs on what the first left in the shared scratch.  Sizes whose scratch would
exceed the stated maximum are refused."""
import ctypes

import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
from gpu_helpers import DEV, II, log, upload

pytestmark = pytest.mark.gpu


def _fn():
    """The entry point and its size query, through the C ABI (ctypes)."""
    lib = cce.lib()
    return lib.cce_forward_no_workspace, lib.cce_forward_no_workspace_max_bytes


def _no_workspace(E, C, t, tile_max):
    f, _ = _fn()
    N, V, D = E.shape[0], C.shape[0], E.shape[1]
    loss = torch.full((N,), float("nan"), device=DEV)
    lse = torch.full((N,), float("nan"), device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    with torch.cuda.device(E.device):
        st = f(ptr(E), ptr(C), ptr(t), N, V, D, cce._lib.dtype_code(E.dtype), II, ptr(loss),
               ptr(lse), ptr(tile_max), ptr(flag),
               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, cce._lib._STATUS.get(st, st)
    return loss, lse, flag


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_workspace_forward_matches_the_workspace_forward(dtype):
    _, max_bytes = _fn()
    assert max_bytes() == 16 << 20
    # the second call is smaller: a different split count and fewer tokens than the first
    for N, V, D, seed in ((5000, 9000, 136, 5), (300, 1100, 72, 6)):
        log(f"[no workspace {dtype}] N={N} V={V} D={D}")
        d = S.small_case(N, D, V, dtype, seed, 3.0, 1.1, 0.1)
        d["targets"][3] = V + 7     # an invalid target: NaN loss and the flag, like cce_forward
        E, C, t = upload(d, dtype)
        assert cce.forward_workspace_bytes(N, V, D, E.dtype) <= max_bytes()
        tm_a, tm_b = cce.tile_max_buffer(E, C), cce.tile_max_buffer(E, C)
        loss_a, lse_a, flag_a = _no_workspace(E, C, t, tm_a)
        flag_b = torch.zeros(1, dtype=torch.int32, device=DEV)
        loss_b, lse_b = cce.cce_forward(E, C, t, II, tile_max=tm_b, err_flag=flag_b)
        torch.cuda.synchronize()
        assert torch.equal(lse_a, lse_b)
        assert torch.equal(loss_a.isnan(), loss_b.isnan()) and bool(loss_a.isnan()[3])
        ok = ~loss_b.isnan()
        assert torch.equal(loss_a[ok], loss_b[ok])
        assert torch.equal(tm_a, tm_b)
        assert int(flag_a.item()) == 1 and int(flag_b.item()) == 1


def test_no_workspace_forward_refuses_sizes_beyond_its_scratch():
    """The scratch holds 16 MiB of partials: 2^21 tokens with one vocabulary range fit exactly,
    256 more do not, and the call is refused on the host (CCE_ERR_WORKSPACE_TOO_SMALL = 3)
    before anything is launched or any pointer is read."""
    f, max_bytes = _fn()
    fake = ctypes.c_void_p(0x1000)
    N = (1 << 21) + 256
    assert cce.forward_workspace_bytes(N, 256, 8, torch.bfloat16) > max_bytes()
    assert f(fake, fake, fake, N, 256, 8, 1, II, fake, fake, None, None, None) == 3
    assert cce.forward_workspace_bytes(1 << 21, 256, 8, torch.bfloat16) == max_bytes()
    # invalid sizes are reported as by cce_forward
    assert f(fake, fake, fake, 16, 0, 8, 1, II, fake, fake, None, None, None) == 1
    assert f(None, None, None, 0, 10, 8, 1, II, None, None, None, None, None) == 0
