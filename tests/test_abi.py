"""The C ABI without a GPU: every declared symbol is exported, the workspace formulas carry
no N x V term, and invalid arguments are rejected on the host before anything is launched."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

F32, BF16 = 0, 1
MIB = 1 << 20


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(cce_\w+)\s*\(", text))
    return sorted(names)


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
    its imports from the HIP runtime are kernel launches, the launch error query, the events of
    the benchmark timing hook (whose end call waits for its own events), and, for the forward
    that takes no workspace, the current device and the device address of its static scratch
    array."""
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
                   "hipEventRecord", "hipEventElapsedTime", "hipEventSynchronize",
                   "hipGetDevice", "hipGetSymbolAddress"}, hip


def test_status_strings(lib):
    assert lib.cce_status_string(0) == b"CCE_OK"
    assert lib.cce_status_string(3) == b"CCE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.cce_status_string(99) == b"CCE_ERR_UNKNOWN"


def g_cap(dt):
    """Largest G store of the backward: two (token block, vocabulary chunk) pairs of at most
    Nc x 8192 entries (Nc = 16384 for bf16 inputs, 8192 for fp32), 512 MiB either way, plus
    their 64 x 64 block flags."""
    nc = 16384 if dt == BF16 else 8192
    return 2 * (nc * 8192 * (2 if dt == BF16 else 4) + (nc // 64) * 128 + 512)


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("gdt", [F32, BF16])
def test_workspace_has_no_tokens_times_vocabulary_term(lib, dt, gdt):
    """Extra device bytes: forward <= 8 bytes x 256 ranges per token; backward <= a constant
    G store (at most 512 MiB) + one float per 256-token tile, + for bf16 gradients the fp32
    running sums, N x D of dE and Vc x D of one chunk's dC.  Nothing grows with N x V."""
    for V, D in ((256000, 2304), (128256, 4096), (32000, 2048), (1000, 64), (10 ** 6, 64)):
        for N in (1, 255, 4096, 8192, 65536, 1 << 20):
            fb = lib.cce_forward_workspace_bytes(N, V, D, dt)
            bb = lib.cce_backward_workspace_bytes(N, V, D, dt, gdt)
            mb = lib.cce_loss_mean_workspace_bytes(N, V, D, dt, gdt)
            acc = (N * D * 4 + 8192 * D * 4 + 512) if gdt == BF16 else 0
            assert 0 < fb <= 2048 * N + 256
            assert 0 < bb <= g_cap(dt) + (N // 256 + 1) * 4 + 256 + acc
            assert fb + bb < mb <= fb + bb + 8 * (N + 64) + 512
    # the logits of one config-sized problem would be 4 N V bytes; the workspace is far below
    N, V, D = 8192, 256000, 2304
    total = lib.cce_loss_mean_workspace_bytes(N, V, D, BF16, F32)
    assert total < 4 * N * V / 20


@pytest.mark.parametrize("dt", [F32, BF16])
def test_backward_workspace_stops_growing_with_tokens(lib, dt):
    """Past one token block the G store no longer grows: with fp32 gradients the backward
    workspace grows only by the 4 bytes per 256-token tile of the LSE minima, and bf16
    gradients add exactly the fp32 dE running sum (N x D floats) and one chunk's dC running sum
    (Vc x D floats)."""
    V, D = 256000, 2304
    nc = lib.cce_backward_token_block(1 << 20, V, D, dt)
    assert nc == (16384 if dt == BF16 else 8192)
    big = [lib.cce_backward_workspace_bytes(N, V, D, dt, F32) for N in (4 * nc, 16 * nc)]
    assert big[1] - big[0] <= (12 * nc // 256) * 4 + 256
    assert big[0] <= g_cap(dt) + 64 * 1024
    for N in (nc // 2, 4 * nc):
        f32 = lib.cce_backward_workspace_bytes(N, V, D, dt, F32)
        b16 = lib.cce_backward_workspace_bytes(N, V, D, dt, BF16)
        rnd = lambda x: -(-x // 256) * 256
        extra = rnd(N * D * 4) + (rnd(8192 * D * 4) if N > nc else 0)
        assert b16 - f32 == extra


def test_workspace_at_the_benchmark_shapes(lib):
    """The backward workspace (fp32 gradients) at the Gemma-2-2B-shaped head (N = 8192,
    V = 256000) is G of two 8192 x 8192 pairs, 256 MiB and flags; at the long-sequence shape
    (N = 65536, V = 32000) four token blocks of 16384 keep it at 512 MiB and flags."""
    g2 = lib.cce_backward_workspace_bytes(8192, 256000, 2304, BF16, F32)
    ls = lib.cce_backward_workspace_bytes(65536, 32000, 2048, BF16, F32)
    assert 256 * MIB < g2 <= 256 * MIB + 64 * 1024
    assert 512 * MIB < ls <= 512 * MIB + 128 * 1024


def test_plan_introspection(lib):
    assert lib.cce_forward_splits(8192, 256000, 2304, 1) == 8
    assert lib.cce_forward_splits(256, 1000, 64, 0) == 4
    # 1000 vocabulary tiles in 32 balanced chunks of 31 or 32 tiles
    assert lib.cce_backward_chunk(8192, 256000, 2304, 1) == 8192
    assert lib.cce_backward_chunk(8192, 20000, 72, 1) == 27 * 256    # 79 tiles in 3 chunks
    assert lib.cce_backward_chunk(256, 1000, 64, 0) == 1024
    # token blocks: balanced, at most 64 tiles (bf16) or 32 (fp32)
    assert lib.cce_backward_token_block(8192, 256000, 2304, 1) == 8192
    assert lib.cce_backward_token_block(65536, 32000, 2048, 1) == 16384
    assert lib.cce_backward_token_block(20000, 1000, 64, 1) == 40 * 256  # 79 tiles in 2 blocks
    assert lib.cce_backward_token_block(20000, 1000, 64, 0) == 27 * 256  # ... in 3 blocks


def test_invalid_sizes_give_zero_workspace(lib):
    assert lib.cce_forward_workspace_bytes(-1, 10, 8, 1) == 0
    assert lib.cce_forward_workspace_bytes(10, 0, 8, 1) == 0
    assert lib.cce_backward_workspace_bytes(10, 10, 12, 1, 0) == 0   # D % 8 for bf16
    assert lib.cce_backward_workspace_bytes(10, 10, 12, 0, 0) > 0    # D % 4 for fp32
    assert lib.cce_forward_workspace_bytes(10, 10, 8, 7) == 0        # unknown dtype
    assert lib.cce_backward_workspace_bytes(10, 10, 8, 1, 3) == 0    # unknown gradient dtype
    assert lib.cce_loss_mean_workspace_bytes(10, 10, 8, 1, 3) == 0


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
    assert lib.cce_backward_workspace_bytes(16, (1 << 24) + 1, 64, 1, 0) == 0
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
    ok_ws = lib.cce_backward_workspace_bytes(16, 100, 64, 1, 0)
    base = dict(dl=_fake(9), stride=1, E=_fake(1), C=_fake(2), t=_fake(3), lse=_fake(4),
                tm=None, N=16, V=100, D=64, dt=1, ii=-100, eps=0.0, floor=0.0, dE=_fake(5),
                dC=_fake(6), gdt=0, ws=_fake(7), wsb=ok_ws, sk=None, st=None)
    call = lambda **k: lib.cce_backward(*dict(base, **k).values())
    assert call(gdt=2) == 1
    assert call(eps=-1.0) == 1
    assert call(eps=float("inf")) == 1
    assert call(eps=float("nan")) == 1
    assert call(floor=-1e-6) == 1
    assert call(floor=float("inf")) == 1
    assert call(floor=float("nan")) == 1
    assert call(stride=2) == 1
    assert call(dl=None) == 1
    assert call(lse=None) == 1
    assert call(wsb=ok_ws - 1) == 3
    # bf16 gradients need the fp32 running sum of dE: the fp32-gradient workspace is too small
    assert call(gdt=1) == 3
    assert call(D=4) == 1
    for name in ("E", "C", "dE", "dC", "ws"):
        assert call(**{name: ctypes.c_void_p(0x2004)}) == 1
    assert call(tm=ctypes.c_void_p(0x2002)) == 1
    assert call(N=0, dC=ctypes.c_void_p(0x2004)) == 1


def test_loss_mean_validation(lib):
    ok_ws = lib.cce_loss_mean_workspace_bytes(16, 100, 64, 1, 1)
    base = dict(E=_fake(1), C=_fake(2), t=_fake(3), N=16, V=100, D=64, dt=1, ii=-100, eps=0.0,
                floor=0.0, mean=_fake(4), nv=None, dE=_fake(5), dC=_fake(6), gdt=1,
                ws=_fake(7), wsb=ok_ws, err=None, sk=None, st=None)
    call = lambda **k: lib.cce_loss_mean(*dict(base, **k).values())
    assert call(gdt=-1) == 1
    assert call(mean=None) == 1
    assert call(wsb=ok_ws - 1) == 3
    assert call(eps=-0.5) == 1
    assert call(floor=-0.5) == 1
    for name in ("E", "C", "dE", "dC", "ws"):
        assert call(**{name: ctypes.c_void_p(0x3002)}) == 1
    assert ok_ws >= (lib.cce_forward_workspace_bytes(16, 100, 64, 1)
                     + lib.cce_backward_workspace_bytes(16, 100, 64, 1, 1))


def test_binding_requires_gpu_tensors():
    import torch
    import linear_cross_entropy_cce_amd as cce
    E = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cce.cce_forward(E, E, torch.zeros(4, dtype=torch.int64))


def test_no_workspace_forward_refuses_on_the_host(lib):
    """The forward without workspace refuses, before touching any pointer or the GPU, problems
    whose scratch exceeds its 16 MiB (WORKSPACE_TOO_SMALL = 3), reports invalid sizes as
    cce_forward does, and treats N = 0 as a no-op."""
    assert lib.cce_forward_no_workspace_max_bytes() == 16 << 20
    N = (1 << 21) + 256
    assert lib.cce_forward_workspace_bytes(N, 256, 8, BF16) > 16 << 20
    assert lib.cce_forward_workspace_bytes(1 << 21, 256, 8, BF16) == 16 << 20
    f = lambda n, v, d, dt: lib.cce_forward_no_workspace(_fake(1), _fake(2), _fake(3), n, v, d,
                                                         dt, -100, _fake(4), _fake(5), None,
                                                         None, None)
    assert f(N, 256, 8, BF16) == 3
    assert f(16, 0, 8, BF16) == 1
    assert f(16, 100, 12, BF16) == 1
    assert f(16, 1 << 25, 8, BF16) == 2
    assert lib.cce_forward_no_workspace(None, None, None, 0, 10, 8, BF16, -100, None, None,
                                        None, None, None) == 0
