"""ctypes binding of libcce (include/cce.h, include/cce_timing.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of libcce.so; this module only turns torch
tensors into device pointers, sizes and the current HIP stream, allocates outputs and
workspaces with torch (device memory plumbing) and maps status codes to exceptions.  There is
no CPU fallback: if libcce.so is missing or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcce.so")

CCE_F32, CCE_BF16 = 0, 1
_STATUS = {0: "CCE_OK", 1: "CCE_ERR_INVALID_ARGUMENT", 2: "CCE_ERR_UNSUPPORTED",
           3: "CCE_ERR_WORKSPACE_TOO_SMALL", 4: "CCE_ERR_HIP"}

_lib = None

_c_ptr, _i64, _sz, _i32, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int, ctypes.c_float

# name -> (restype, argtypes); the C ABI declared in include/cce.h
SIGNATURES = {
    "cce_status_string": (ctypes.c_char_p, [_i32]),
    "cce_forward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "cce_backward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "cce_loss_mean_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "cce_forward_splits": (_i64, [_i64, _i64, _i64, _i32]),
    "cce_backward_chunk": (_i64, [_i64, _i64, _i64, _i32]),
    "cce_backward_token_block": (_i64, [_i64, _i64, _i64, _i32]),
    "cce_tile_max_count": (_i64, [_i64, _i64, _i64, _i32]),
    "cce_forward": (_i32, [_c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i32, _i64, _c_ptr, _c_ptr,
                           _c_ptr, _c_ptr, _sz, _c_ptr, _c_ptr]),
    "cce_backward": (_i32, [_c_ptr, _i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _i64, _i64,
                            _i64, _i32, _i64, _f32, _f32, _c_ptr, _c_ptr, _i32, _c_ptr, _sz,
                            _c_ptr, _c_ptr]),
    "cce_loss_mean": (_i32, [_c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i32, _i64, _f32, _f32,
                             _c_ptr, _c_ptr, _c_ptr, _c_ptr, _i32, _c_ptr, _sz, _c_ptr, _c_ptr,
                             _c_ptr]),
    "cce_forward_no_workspace": (_i32, [_c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i32, _i64,
                                        _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "cce_forward_no_workspace_max_bytes": (_sz, []),
    "cce_forward_shard": (_i32, [_c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i32, _i64, _i64,
                                 _c_ptr, _c_ptr, _c_ptr, _c_ptr, _sz, _c_ptr]),
    "cce_merge_shards": (_i32, [_c_ptr, _c_ptr, _i64, _i64, _c_ptr, _i64, _i64, _c_ptr, _c_ptr,
                                _c_ptr, _c_ptr]),
    "cce_backward_shard": (_i32, [_c_ptr, _i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _i64,
                                  _i64, _i64, _i32, _i64, _i64, _f32, _f32, _c_ptr, _c_ptr,
                                  _i32, _c_ptr, _sz, _c_ptr, _c_ptr]),
    "cce_timing_begin": (_i32, [ctypes.c_uint32, ctypes.c_int32]),
    "cce_timing_end": (_i32, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int64)]),
}

KERNEL_KINDS = ("fwd_lse", "fwd_finish", "bwd_g", "bwd_fused", "aux")


class CCEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Loads libcce.so once.  torch is imported first so that the HIP runtime it carries (same
    soname as the one libcce links) is the one both use."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                               "linear_cross_entropy_cce_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return CCE_BF16
    if t == torch.float32:
        return CCE_F32
    raise TypeError(f"E and C must be bfloat16 or float32, not {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CCEError(fn, status)


def _check_inputs(E, C, targets):
    for name, t in (("E", E), ("C", C), ("targets", targets)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != E.device:
            raise ValueError(f"{name} is on {t.device}, E on {E.device}")
    if E.dim() != 2 or C.dim() != 2 or E.shape[1] != C.shape[1]:
        raise ValueError(f"E [N,D] and C [V,D] expected, got {tuple(E.shape)}, {tuple(C.shape)}")
    if E.dtype != C.dtype:
        raise TypeError("E and C must have the same dtype")
    if targets.dtype != torch.int64 or targets.shape != (E.shape[0],):
        raise ValueError("targets must be int64 [N]")
    return E.shape[0], C.shape[0], E.shape[1], dtype_code(E.dtype)


def _check_vec(name, t, n, dtype, dev):
    """A caller-supplied per-token array: contiguous, dtype, [n], on the inputs' device."""
    if (t.dtype != dtype or tuple(t.shape) != (n,) or not t.is_contiguous() or not t.is_cuda
            or t.device != dev):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor [{n}] on {dev}")


def _check_flags(dev, err_flag=None, skip_stats=None):
    """The optional device outputs: err_flag int32 [1], skip_stats int64 [2]."""
    if err_flag is not None:
        _check_vec("err_flag", err_flag, 1, torch.int32, dev)
    if skip_stats is not None:
        _check_vec("skip_stats", skip_stats, 2, torch.int64, dev)


def forward_workspace_bytes(N: int, V: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().cce_forward_workspace_bytes(N, V, D, dtype_code(dtype)))


def backward_workspace_bytes(N: int, V: int, D: int, dtype: torch.dtype,
                             grad_dtype: torch.dtype = torch.float32) -> int:
    return int(lib().cce_backward_workspace_bytes(N, V, D, dtype_code(dtype),
                                                  dtype_code(grad_dtype)))


def loss_mean_workspace_bytes(N: int, V: int, D: int, dtype: torch.dtype,
                              grad_dtype: torch.dtype = torch.float32) -> int:
    return int(lib().cce_loss_mean_workspace_bytes(N, V, D, dtype_code(dtype),
                                                   dtype_code(grad_dtype)))


def forward_splits(N: int, V: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().cce_forward_splits(N, V, D, dtype_code(dtype)))


def backward_chunk(N: int, V: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().cce_backward_chunk(N, V, D, dtype_code(dtype)))


def backward_token_block(N: int, V: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().cce_backward_token_block(N, V, D, dtype_code(dtype)))


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _workspace_arg(ws, nbytes: int, dev) -> torch.Tensor:
    """The caller's workspace (its size is checked by the library), or a new one."""
    if ws is None:
        return workspace(nbytes, dev)
    if not ws.is_cuda or ws.device != dev or not ws.is_contiguous():
        raise ValueError(f"the workspace must be a contiguous tensor on {dev}")
    return ws


def tile_max_count(N: int, V: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().cce_tile_max_count(N, V, D, dtype_code(dtype)))


def tile_max_buffer(E, C) -> torch.Tensor:
    """An fp32 device buffer for the forward's tile maxima (cce_forward(tile_max=...)), to be
    passed on to cce_backward(tile_max=...)."""
    n = tile_max_count(E.shape[0], C.shape[0], E.shape[1], E.dtype)
    return torch.empty(max(n, 1), dtype=torch.float32, device=E.device)


def _check_tile_max(t, N, V, D, dt, dev):
    if t is None:
        return
    n = int(lib().cce_tile_max_count(N, V, D, dt))
    if (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda or t.device != dev
            or t.numel() < n):
        raise ValueError(f"tile_max must be a contiguous float32 tensor of at least {n} "
                         f"elements on {dev}")


def cce_forward(E, C, targets, ignore_index: int = -100, *, loss=None, lse=None, tile_max=None,
                ws=None, err_flag=None, stream=None):
    """Per-token loss and LSE (fp32 [N]).  Returns (loss, lse).  tile_max (optional, from
    tile_max_buffer) receives the tile maxima that let cce_backward skip negligible tiles."""
    N, V, D, dt = _check_inputs(E, C, targets)
    dev = E.device
    loss = torch.empty(N, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    _check_vec("loss", loss, N, torch.float32, dev)
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_tile_max(tile_max, N, V, D, dt, dev)
    need = lib().cce_forward_workspace_bytes(N, V, D, dt)
    ws = _workspace_arg(ws, need, dev)
    _check_flags(dev, err_flag=err_flag)
    with torch.cuda.device(dev):
        _check("cce_forward", lib().cce_forward(
            _ptr(E), _ptr(C), _ptr(targets), N, V, D, dt, ignore_index, _ptr(loss), _ptr(lse),
            _ptr(tile_max), _ptr(ws), ws.numel() * ws.element_size(), _ptr(err_flag),
            _stream(stream)))
    return loss, lse


def cce_forward_no_workspace(E, C, targets, ignore_index: int = -100, *, loss=None, lse=None,
                             tile_max=None, err_flag=None, stream=None):
    """cce_forward for callers that cannot allocate: no workspace (the library's static 16 MiB
    scratch of the current device instead), so no allocation happens when loss and lse are
    passed in.  Calls that overlap on one GPU share that scratch and must be ordered."""
    N, V, D, dt = _check_inputs(E, C, targets)
    dev = E.device
    loss = torch.empty(N, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    _check_vec("loss", loss, N, torch.float32, dev)
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_tile_max(tile_max, N, V, D, dt, dev)
    _check_flags(dev, err_flag=err_flag)
    with torch.cuda.device(dev):
        _check("cce_forward_no_workspace", lib().cce_forward_no_workspace(
            _ptr(E), _ptr(C), _ptr(targets), N, V, D, dt, ignore_index, _ptr(loss), _ptr(lse),
            _ptr(tile_max), _ptr(err_flag), _stream(stream)))
    return loss, lse


def forward_no_workspace_max_bytes() -> int:
    return int(lib().cce_forward_no_workspace_max_bytes())


def _grad_outputs(N, V, D, dev, grad_dtype, dE, dC):
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    dE = torch.empty((N, D), dtype=gdt, device=dev) if dE is None else dE
    dC = torch.empty((V, D), dtype=gdt, device=dev) if dC is None else dC
    for name, g, shape in (("dE", dE, (N, D)), ("dC", dC, (V, D))):
        if (g.dtype != gdt or tuple(g.shape) != shape or not g.is_contiguous() or not g.is_cuda
                or g.device != dev):
            raise ValueError(f"{name} must be a contiguous {gdt} tensor of shape {shape} on {dev}")
    return dE, dC, dtype_code(gdt)


def cce_backward(dloss, E, C, targets, lse, ignore_index: int = -100, filter_eps: float = 0.0,
                 *, entry_floor: float = 0.0, tile_max=None, dE=None, dC=None, grad_dtype=None,
                 ws=None, skip_stats=None, stream=None):
    """dE [N,D] and dC [V,D] in grad_dtype (torch.float32 by default, or torch.bfloat16).
    dloss: fp32 [N], or a 1-element tensor (scalar).  tile_max: the forward's tile maxima for
    the same E, C and targets, or None.  entry_floor: 0 (off) or the softmax value below which
    non-target entries of the kept blocks are dropped."""
    N, V, D, dt = _check_inputs(E, C, targets)
    dev = E.device
    if dloss.dtype != torch.float32 or not dloss.is_cuda or dloss.device != dev:
        raise ValueError(f"dloss must be a float32 tensor on {dev}")
    stride = 0 if dloss.numel() == 1 and N != 1 else 1
    if stride == 1 and dloss.shape != (N,):
        raise ValueError("dloss must have N elements or one")
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_tile_max(tile_max, N, V, D, dt, dev)
    dE, dC, gcode = _grad_outputs(N, V, D, dev, grad_dtype, dE, dC)
    need = lib().cce_backward_workspace_bytes(N, V, D, dt, gcode)
    ws = _workspace_arg(ws, need, dev)
    _check_flags(dev, skip_stats=skip_stats)
    with torch.cuda.device(dev):
        _check("cce_backward", lib().cce_backward(
            _ptr(dloss), stride, _ptr(E), _ptr(C), _ptr(targets), _ptr(lse), _ptr(tile_max), N,
            V, D, dt, ignore_index, float(filter_eps), float(entry_floor), _ptr(dE), _ptr(dC),
            gcode, _ptr(ws), ws.numel() * ws.element_size(), _ptr(skip_stats),
            _stream(stream)))
    return dE, dC


def cce_loss_mean(E, C, targets, ignore_index: int = -100, filter_eps: float = 0.0, *,
                  entry_floor: float = 0.0, dE=None, dC=None, grad_dtype=None, ws=None,
                  err_flag=None, skip_stats=None, stream=None):
    """Mean loss over non-ignored tokens and its gradients (in grad_dtype, fp32 by default).
    Returns (mean[1], n_valid[1], dE, dC) as device tensors."""
    N, V, D, dt = _check_inputs(E, C, targets)
    dev = E.device
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    dE, dC, gcode = _grad_outputs(N, V, D, dev, grad_dtype, dE, dC)
    need = lib().cce_loss_mean_workspace_bytes(N, V, D, dt, gcode)
    ws = _workspace_arg(ws, need, dev)
    _check_flags(dev, err_flag=err_flag, skip_stats=skip_stats)
    with torch.cuda.device(dev):
        _check("cce_loss_mean", lib().cce_loss_mean(
            _ptr(E), _ptr(C), _ptr(targets), N, V, D, dt, ignore_index, float(filter_eps),
            float(entry_floor), _ptr(mean), _ptr(n_valid), _ptr(dE), _ptr(dC), gcode, _ptr(ws),
            ws.numel() * ws.element_size(), _ptr(err_flag), _ptr(skip_stats), _stream(stream)))
    return mean, n_valid, dE, dC


def cce_forward_shard(E, C_shard, targets, vocab_offset: int, ignore_index: int = -100, *,
                      lse=None, target_logit=None, tile_max=None, ws=None, stream=None):
    """One vocabulary shard's forward: (lse over the shard's rows, target logit or 0), fp32 [N].
    targets index the full vocabulary; C_shard holds rows [vocab_offset, vocab_offset + V)."""
    N, V, D, dt = _check_inputs(E, C_shard, targets)
    dev = E.device
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    zt = torch.empty(N, dtype=torch.float32, device=dev) if target_logit is None else target_logit
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_vec("target_logit", zt, N, torch.float32, dev)
    _check_tile_max(tile_max, N, V, D, dt, dev)
    need = lib().cce_forward_workspace_bytes(N, V, D, dt)
    ws = _workspace_arg(ws, need, dev)
    with torch.cuda.device(dev):
        _check("cce_forward_shard", lib().cce_forward_shard(
            _ptr(E), _ptr(C_shard), _ptr(targets), N, V, D, dt, ignore_index, int(vocab_offset),
            _ptr(lse), _ptr(zt), _ptr(tile_max), _ptr(ws), ws.numel() * ws.element_size(),
            _stream(stream)))
    return lse, zt


def cce_merge_shards(lse_shards, target_logits, targets, V_total: int, ignore_index: int = -100,
                     *, loss=None, lse=None, err_flag=None, stream=None):
    """Merges [S, N] per-shard LSEs and target logits into (loss, lse), fp32 [N]."""
    S, N = lse_shards.shape
    for name, t in (("lse_shards", lse_shards), ("target_logits", target_logits)):
        if t.dtype != torch.float32 or t.shape != (S, N) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [S, N]")
    if targets.dtype != torch.int64 or targets.shape != (N,) or not targets.is_cuda:
        raise ValueError("targets must be int64 [N] on the GPU")
    dev = lse_shards.device
    loss = torch.empty(N, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    _check_vec("loss", loss, N, torch.float32, dev)
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_flags(dev, err_flag=err_flag)
    with torch.cuda.device(dev):
        _check("cce_merge_shards", lib().cce_merge_shards(
            _ptr(lse_shards), _ptr(target_logits), S, N, _ptr(targets), ignore_index, int(V_total),
            _ptr(loss), _ptr(lse), _ptr(err_flag), _stream(stream)))
    return loss, lse


def cce_backward_shard(dloss, E, C_shard, targets, lse, vocab_offset: int,
                       ignore_index: int = -100, filter_eps: float = 0.0, *,
                       entry_floor: float = 0.0, tile_max=None, dE=None, dC=None,
                       grad_dtype=None, ws=None, skip_stats=None, stream=None):
    """One vocabulary shard's backward with the merged LSE: (this shard's term of dE, the
    shard's rows of dC)."""
    N, V, D, dt = _check_inputs(E, C_shard, targets)
    dev = E.device
    if dloss.dtype != torch.float32 or not dloss.is_cuda or dloss.device != dev:
        raise ValueError(f"dloss must be a float32 tensor on {dev}")
    stride = 0 if dloss.numel() == 1 and N != 1 else 1
    if stride == 1 and dloss.shape != (N,):
        raise ValueError("dloss must have N elements or one")
    _check_vec("lse", lse, N, torch.float32, dev)
    _check_tile_max(tile_max, N, V, D, dt, dev)
    dE, dC, gcode = _grad_outputs(N, V, D, dev, grad_dtype, dE, dC)
    need = lib().cce_backward_workspace_bytes(N, V, D, dt, gcode)
    ws = _workspace_arg(ws, need, dev)
    _check_flags(dev, skip_stats=skip_stats)
    with torch.cuda.device(dev):
        _check("cce_backward_shard", lib().cce_backward_shard(
            _ptr(dloss), stride, _ptr(E), _ptr(C_shard), _ptr(targets), _ptr(lse),
            _ptr(tile_max), N, V, D, dt, ignore_index, int(vocab_offset), float(filter_eps),
            float(entry_floor), _ptr(dE), _ptr(dC), gcode, _ptr(ws), ws.numel() * ws.element_size(),
            _ptr(skip_stats), _stream(stream)))
    return dE, dC


def timing_begin(kinds=KERNEL_KINDS, max_launches: int = 100000) -> None:
    """Starts recording HIP event pairs around launches of the given kernel kinds."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check("cce_timing_begin", lib().cce_timing_begin(mask, max_launches))


def timing_end() -> dict:
    """Stops recording; returns {kind: (total_ms, launches)} for kinds that ran."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_float * n)()
    cnt = (ctypes.c_int64 * n)()
    _check("cce_timing_end", lib().cce_timing_end(ms, cnt))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS) if cnt[i]}
