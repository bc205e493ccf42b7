"""The C ABI without a GPU: every declared symbol is exported, the workspace formulas carry
no N x V term, and invalid arguments are rejected on the host before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cce_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import linear_cross_entropy_cce_amd as cce
    if not os.path.exists(cce.LIB_PATH):
        from linear_cross_entropy_cce_amd import build
        build.build()
    return cce.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_the_header():
    from linear_cross_entropy_cce_amd import _lib
    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_library_imports_no_allocation_copy_or_sync(lib):
    """The library never allocates, copies or clears device memory and never waits on the host:
    its imports from the HIP runtime are kernel launches, the launch error query and the events
    of the benchmark timing hook (whose end call waits for its own events)."""
    import shutil
    import subprocess
    import linear_cross_entropy_cce_amd as cce
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--undefined-only", cce.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    hip = {line.split()[-1].split("@")[0] for line in out.splitlines()
           if line.split() and line.split()[-1].startswith("hip")}
    assert "hipLaunchKernel" in hip
    assert hip <= {"hipLaunchKernel", "hipGetLastError", "hipEventCreate", "hipEventDestroy",
                   "hipEventRecord", "hipEventElapsedTime", "hipEventSynchronize"}, hip


def test_status_strings(lib):
    assert lib.cce_status_string(0) == b"CCE_OK"
    assert lib.cce_status_string(3) == b"CCE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.cce_status_string(99) == b"CCE_ERR_UNKNOWN"


@pytest.mark.parametrize("dt", [0, 1])
def test_workspace_has_no_tokens_times_vocabulary_term(lib, dt):
    """Extra device bytes are bounded by a per-token constant that does not grow with V:
    forward <= 8 bytes x 256 ranges per token, backward <= two chunks of 8192 vocabulary
    columns of G per (padded) token plus their block flags, plus an fp32 dE accumulator and
    one float per 256-token tile."""
    sz = 4 if dt == 0 else 2
    for V, D in ((256000, 2304), (128256, 4096), (32000, 2048), (1000, 64), (10 ** 6, 64)):
        for N in (1, 255, 4096, 8192, 65536):
            pad = -(-N // 256) * 256
            fb = lib.cce_forward_workspace_bytes(N, V, D, dt)
            bb = lib.cce_backward_workspace_bytes(N, V, D, dt)
            mb = lib.cce_loss_mean_workspace_bytes(N, V, D, dt)
            assert 0 < fb <= 2048 * N + 256
            assert 0 < bb <= (2 * (pad * 8192 * sz + pad * 2 + 256) + N * D * 4 + 256
                              + pad // 256 * 4 + 256)
            assert fb + bb < mb <= fb + bb + 8 * (N + 64) + 512
    # the logits of one config-sized problem would be 4 N V bytes; the workspace is far below
    N, V, D = 8192, 256000, 2304
    total = lib.cce_loss_mean_workspace_bytes(N, V, D, 1)
    assert total < 4 * N * V / 20


@pytest.mark.parametrize("dt", [0, 1])
def test_backward_workspace_is_affine_in_tokens(lib, dt):
    """Sweep N over multiples of the 256-token tile at fixed V and D: the backward workspace
    is exactly a + b N, and the slope b does not grow with V (no N x V term)."""
    slopes = {}
    for V in (32000, 256000, 10 ** 6):
        ws = [lib.cce_backward_workspace_bytes(N, V, 2304, dt) for N in (2048, 4096, 8192, 16384)]
        d1, d2, d3 = ws[1] - ws[0], ws[2] - ws[1], ws[3] - ws[2]
        assert d2 == 2 * d1 and d3 == 2 * d2
        slopes[V] = d1 / 2048
    assert slopes[256000] == slopes[10 ** 6]      # chunk width capped: per-token bytes fixed


def test_plan_introspection(lib):
    assert lib.cce_forward_splits(8192, 256000, 2304, 1) == 8
    assert lib.cce_forward_splits(256, 1000, 64, 0) == 4
    assert lib.cce_backward_chunk(8192, 256000, 2304, 1) == 8192
    assert lib.cce_backward_chunk(256, 1000, 64, 0) == 1024


def test_invalid_sizes_give_zero_workspace(lib):
    assert lib.cce_forward_workspace_bytes(-1, 10, 8, 1) == 0
    assert lib.cce_forward_workspace_bytes(10, 0, 8, 1) == 0
    assert lib.cce_backward_workspace_bytes(10, 10, 12, 1) == 0   # D % 8 for bf16
    assert lib.cce_backward_workspace_bytes(10, 10, 12, 0) > 0    # D % 4 for fp32
    assert lib.cce_forward_workspace_bytes(10, 10, 8, 7) == 0     # unknown dtype


def _fake(n=1):
    return ctypes.c_void_p(0x1000 * n)   # never dereferenced: calls below fail validation


def test_forward_validation(lib):
    ok_ws = lib.cce_forward_workspace_bytes(16, 100, 64, 1)
    args = lambda **k: dict(dict(E=_fake(1), C=_fake(2), t=_fake(3), N=16, V=100, D=64, dt=1,
                                 ii=-100, loss=_fake(4), lse=_fake(5), tm=None, ws=_fake(6),
                                 wsb=ok_ws, err=None, st=None), **k)
    call = lambda a: lib.cce_forward(a["E"], a["C"], a["t"], a["N"], a["V"], a["D"], a["dt"],
                                     a["ii"], a["loss"], a["lse"], a["tm"], a["ws"], a["wsb"],
                                     a["err"], a["st"])
    assert call(args(N=-1)) == 1
    assert call(args(V=0)) == 1
    assert call(args(D=60)) == 1
    assert call(args(dt=5)) == 1
    assert call(args(E=None)) == 1
    assert call(args(loss=None)) == 1
    assert call(args(wsb=ok_ws - 1)) == 3
    assert call(args(N=1 << 25)) == 2
    assert call(args(V=(1 << 24) + 1)) == 2        # beyond the kernels' limits: unsupported
    assert call(args(D=65536 + 8)) == 2
    assert lib.cce_forward_workspace_bytes(16, 100, 65536 + 8, 1) == 0
    assert lib.cce_backward_workspace_bytes(16, (1 << 24) + 1, 64, 1) == 0
    assert lib.cce_forward_workspace_bytes(16, 1 << 24, 65536, 1) > 0   # the limits themselves
    assert call(args(N=0, E=None, C=None, t=None, loss=None, lse=None, ws=None)) == 0
    for name in ("E", "C", "ws"):                      # 16-byte vectors: misaligned -> rejected
        assert call(args(**{name: ctypes.c_void_p(0x1008)})) == 1
    assert call(args(tm=ctypes.c_void_p(0x1002))) == 1  # tile maxima: fp32, 4-byte aligned


def test_tile_max_count(lib):
    assert lib.cce_tile_max_count(8192, 256000, 2304, 1) == 32 * 1000 * 8
    assert lib.cce_tile_max_count(1, 1, 8, 1) == 8
    assert lib.cce_tile_max_count(0, 300, 8, 1) == 1 * 2 * 8
    assert lib.cce_tile_max_count(16, 100, 60, 1) == 0              # invalid sizes


def test_backward_validation(lib):
    ok_ws = lib.cce_backward_workspace_bytes(16, 100, 64, 1)
    base = dict(dl=_fake(9), stride=1, E=_fake(1), C=_fake(2), t=_fake(3), lse=_fake(4),
                tm=None, N=16, V=100, D=64, dt=1, ii=-100, eps=0.0, dE=_fake(5), dC=_fake(6),
                gdt=0, ws=_fake(7), wsb=ok_ws, sk=None, st=None)
    call = lambda **k: lib.cce_backward(*dict(base, **k).values())
    assert call(gdt=2) == 1
    assert call(eps=-1.0) == 1
    assert call(eps=float("inf")) == 1
    assert call(eps=float("nan")) == 1
    assert call(stride=2) == 1
    assert call(dl=None) == 1
    assert call(lse=None) == 1
    assert call(wsb=ok_ws - 1) == 3
    assert call(D=4) == 1
    for name in ("E", "C", "dE", "dC", "ws"):
        assert call(**{name: ctypes.c_void_p(0x2004)}) == 1
    assert call(tm=ctypes.c_void_p(0x2002)) == 1
    assert call(N=0, dC=ctypes.c_void_p(0x2004)) == 1


def test_loss_mean_validation(lib):
    ok_ws = lib.cce_loss_mean_workspace_bytes(16, 100, 64, 1)
    base = dict(E=_fake(1), C=_fake(2), t=_fake(3), N=16, V=100, D=64, dt=1, ii=-100, eps=0.0,
                mean=_fake(4), nv=None, dE=_fake(5), dC=_fake(6), gdt=1, ws=_fake(7),
                wsb=ok_ws, err=None, sk=None, st=None)
    call = lambda **k: lib.cce_loss_mean(*dict(base, **k).values())
    assert call(gdt=-1) == 1
    assert call(mean=None) == 1
    assert call(wsb=ok_ws - 1) == 3
    assert call(eps=-0.5) == 1
    for name in ("E", "C", "dE", "dC", "ws"):
        assert call(**{name: ctypes.c_void_p(0x3002)}) == 1
    assert ok_ws >= (lib.cce_forward_workspace_bytes(16, 100, 64, 1)
                     + lib.cce_backward_workspace_bytes(16, 100, 64, 1))


def test_binding_requires_gpu_tensors():
    import torch
    import linear_cross_entropy_cce_amd as cce
    E = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cce.cce_forward(E, E, torch.zeros(4, dtype=torch.int64))
