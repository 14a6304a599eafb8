"""MI355X-native chunkwise retention and causal linear attention.

Thin Python binding over ``libretention.so`` (C ABI in ``include/retention.h``).
This module only marshals arguments: it checks that tensors are CUDA (HIP)
tensors of the right dtype and layout, allocates outputs with PyTorch when the
caller does not pass them, and hands raw device pointers plus the current HIP
stream to the library.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  If the library is not built, every
call raises.

Functions
---------
retention_fwd(q, k, v, gamma, chunk=64, initial_state=None) -> (out, final_state)
retention_fwd_noalloc(q, k, v, gamma, chunk=64) -> (out, final_state)   (no workspace: library device array)
retention_decode_step(q, k, v, gamma, state)   -> out      (state updated in place)
linear_attn_fwd(q, k, v, phi="elu1", eps=1e-6) -> out
linear_attn_fwd(..., initial_state=(S, z), return_state=True) -> (out, S, z)
linear_attn_decode_step(q, k, v, S, z, eps=1e-6) -> out   (S, z updated in place)
retention_bwd(q, k, v, gamma, dout, chunk=64)  -> (dq, dk, dv); fwd_workspace= reuses a forward's states
retention_fwd_normalized(q, k, v, gamma, norm="group", eps=1e-5) -> out   (bf16 or fp32)
retention(q, k, v, gamma, chunk=64)            -> out, differentiable (torch.autograd)
gla_fwd(q, k, v, log_gate)                     -> (out, final_state)   (fp32 or bf16 q/k/v, fp32 gates)
retention_fwd_workspace_bytes(B, H, T, dk, dv, chunk, dtype) -> int
linear_attn_workspace_bytes(B, H, T, dk, dv, dtype)          -> int
set_plan_override(path=None, segments=None, walk_nt=None, lin_chunk=None)   (this thread's calls)
plan_override(...)                             context manager around set_plan_override

The two forwards take an optional ``workspace=`` uint8 tensor for the
segment states of the bf16 paths; without one, the binding takes it from
PyTorch's allocator for the call.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import numpy as np
import torch

__all__ = ["retention_fwd", "retention_fwd_noalloc", "retention_bwd", "retention", "retention_decode_step", "linear_attn_fwd",
           "linear_attn_decode_step", "retention_bwd_workspace_bytes", "retention_fwd_normalized",
           "retention_fwd_normalized_workspace_bytes", "gla_fwd", "RET_NORM_ROWSUM", "RET_NORM_GROUP",
           "retention_fwd_workspace_bytes",
           "linear_attn_workspace_bytes", "RetentionError", "set_plan_override", "plan_override",
           "library_path", "load_library", "abi_version", "last_error"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libretention.so")
_DEBUG_LIB_PATH = os.path.join(_HERE, "libretention_debug.so")
_lock = threading.Lock()
_lib = None
_dlib = None

RET_F32 = 0
RET_BF16 = 1
RET_PHI_ELU1 = 1
RET_NORM_ROWSUM = 1
RET_NORM_GROUP = 2
RET_PATH = {None: 0, "auto": 0, "slice": 1, "segment": 2}
ERRORS = {
    -1: "RET_ERR_NULL", -2: "RET_ERR_SHAPE", -3: "RET_ERR_DTYPE", -4: "RET_ERR_CHUNK",
    -5: "RET_ERR_GAMMA", -6: "RET_ERR_PHI", -7: "RET_ERR_ALIGN", -8: "RET_ERR_ALIAS",
    -9: "RET_ERR_WORKSPACE", -10: "RET_ERR_HIP",
}
MAX_HEADS = 256


class RetentionError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def _declare(lib):
    """Argument and result types of the C ABI on a loaded library."""
    vp, fp, i, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int, ctypes.c_size_t
    lib.retention_fwd.argtypes = [vp, vp, vp, fp, i, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.retention_fwd.restype = i
    lib.retention_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_fwd_workspace_bytes.restype = sz
    lib.linear_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.linear_attn_workspace_bytes.restype = sz
    lib.retention_decode_step.argtypes = [vp, vp, vp, fp, vp, vp, i, i, i, i, i, vp]
    lib.retention_decode_step.restype = i
    lib.linear_attn_fwd.argtypes = [vp, vp, vp, i, vp, i, i, i, i, i, i, ctypes.c_float, vp, sz, vp]
    lib.retention_fwd_noalloc.argtypes = [vp, vp, vp, fp, i, vp, vp, i, i, i, i, i, i, vp]
    lib.retention_fwd_noalloc.restype = i
    lib.retention_fwd_from_state.argtypes = [vp, vp, vp, fp, i, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.retention_fwd_from_state.restype = i
    lib.linear_attn_fwd_from_state.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                               ctypes.c_float, vp, sz, vp]
    lib.linear_attn_fwd_from_state.restype = i
    lib.linear_attn_decode_step.argtypes = [vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, ctypes.c_float, vp]
    lib.linear_attn_decode_step.restype = i
    lib.retention_bwd.argtypes = [vp, vp, vp, fp, i, vp, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.retention_bwd.restype = i
    lib.retention_bwd_from_fwd.argtypes = [vp, vp, vp, fp, i, vp, vp, sz, vp, vp, vp, i, i, i, i, i, i, vp,
                                           sz, vp]
    lib.retention_bwd_from_fwd.restype = i
    lib.retention_fwd_normalized.argtypes = [vp, vp, vp, fp, i, i, ctypes.c_float, vp, i, i, i, i, i, i, vp,
                                             sz, vp]
    lib.retention_fwd_normalized.restype = i
    lib.retention_fwd_normalized_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_fwd_normalized_workspace_bytes.restype = sz
    lib.gla_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.gla_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gla_fwd_workspace_bytes.restype = sz
    lib.gla_fwd.restype = i
    lib.retention_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_bwd_workspace_bytes.restype = sz
    lib.linear_attn_fwd.restype = i
    lib.retention_last_error.argtypes = []
    lib.retention_last_error.restype = ctypes.c_char_p
    lib.retention_abi_version.argtypes = []
    lib.retention_abi_version.restype = i
    lib.retention_set_plan_override.argtypes = [i, i, i, i]
    lib.retention_set_plan_override.restype = i
    return lib


def load_debug_library():
    """Load libretention_debug.so, the LDS hazard self-check build (-DRET_DEBUG:
    every LDS buffer that has gone dead is overwritten with NaN words until it
    is refilled).  A separate handle with the same C ABI; the functions of this
    module keep using the normal build."""
    global _dlib
    with _lock:
        if _dlib is None:
            if not os.path.exists(_DEBUG_LIB_PATH):
                raise RuntimeError(f"{_DEBUG_LIB_PATH} is missing: build it with "
                                   "`python -m retention_chunkwise_amd._build --debug`")
            _dlib = _declare(ctypes.CDLL(_DEBUG_LIB_PATH))
        return _dlib


def load_library():
    """Load libretention.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with `python -m retention_chunkwise_amd._build` "
                    "(or __graft_entry__.build()); there is no non-HIP fallback")
            _lib = _declare(ctypes.CDLL(_LIB_PATH))
        return _lib


def abi_version() -> int:
    return int(load_library().retention_abi_version())


def last_error() -> str:
    return load_library().retention_last_error().decode()


def _raise(rc: int):
    if rc != 0:
        raise RetentionError(rc, last_error())


def set_plan_override(path=None, segments=None, walk_nt=None, lin_chunk=None) -> None:
    """Fix parts of the library's execution plan for later calls made from
    the calling thread (retention_set_plan_override in the C ABI); with no
    arguments the automatic plan is restored.  path: "slice" | "segment" |
    None; segments: the segment count per sequence; walk_nt: value-slice width
    of the slice path in 16-column tiles; lin_chunk: 64 | 128.  Results do
    not change beyond rounding."""
    if path not in RET_PATH:
        raise ValueError(f"path must be one of {sorted(k for k in RET_PATH if k)} or None")
    _raise(load_library().retention_set_plan_override(RET_PATH[path], int(segments or 0), int(walk_nt or 0),
                                                      int(lin_chunk or 0)))


@contextlib.contextmanager
def plan_override(**kw):
    """``with plan_override(segments=4): ...`` -- set_plan_override for the
    block, then the automatic plan again."""
    set_plan_override(**kw)
    try:
        yield
    finally:
        set_plan_override()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RET_F32
    if t.dtype == torch.bfloat16:
        return RET_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_dev(name: str, t: torch.Tensor, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def _gamma_array(gamma, H: int):
    g = np.ascontiguousarray(np.asarray(
        gamma.detach().cpu().numpy() if isinstance(gamma, torch.Tensor) else gamma,
        dtype=np.float32).reshape(-1))
    if g.size == 1 and H > 1:
        g = np.full(H, g[0], dtype=np.float32)
    if g.size != H:
        raise ValueError(f"gamma must have {H} entries (got {g.size})")
    return (ctypes.c_float * H)(*g.tolist())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(nbytes: int, device, given=None):
    """Scratch for the segment-split paths: the caller's uint8 tensor when one
    is given (the library checks its size), else one from PyTorch's allocator
    on the current stream (returned to that stream's pool after the call is
    enqueued)."""
    if given is not None:
        _check_dev("workspace", given, torch.uint8)
        return given, given.numel()
    if nbytes <= 0:
        return None, 0
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device), int(nbytes)


def retention_fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                                  dtype=torch.bfloat16) -> int:
    """Bytes of device workspace retention_fwd needs for these sizes (0: none)."""
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_fwd_workspace_bytes(B, H, T, dk, dv, int(chunk), code))


def retention_fwd_normalized_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                                             dtype=torch.bfloat16) -> int:
    """Bytes of device workspace retention_fwd_normalized needs (0: none)."""
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_fwd_normalized_workspace_bytes(B, H, T, dk, dv, int(chunk), code))


def retention_bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                                  dtype=torch.bfloat16) -> int:
    """Bytes of device workspace retention_bwd needs for these sizes (0: none)."""
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().retention_bwd_workspace_bytes(B, H, T, dk, dv, int(chunk), code))


def linear_attn_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype=torch.bfloat16) -> int:
    """Bytes of device workspace linear_attn_fwd needs for these sizes (0: none)."""
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    return int(load_library().linear_attn_workspace_bytes(B, H, T, dk, dv, code))


def _ptr(t):
    return t.data_ptr() if t is not None else None


def retention_fwd(q, k, v, gamma, chunk: int = 64, out=None, final_state=None,
                  want_state: bool = True, workspace=None, initial_state=None):
    """Chunkwise causal retention, from a zero state or from initial_state.

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (float32 or bfloat16, same dtype, on the
    GPU); gamma: H decay values in (0, 1].  Returns (out, final_state) with
    out [B,H,T,dv] in the input dtype and final_state [B,H,dk,dv] float32
    (None if want_state is False and none was passed).  initial_state:
    optional [B,H,dk,dv] float32 state after earlier tokens (e.g. a previous
    call's final_state; it must not be the final_state buffer of this call).
    workspace: optional uint8 GPU tensor of at least
    retention_fwd_workspace_bytes(...) bytes; one is allocated per call when it
    is omitted.
    """
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    if final_state is None and want_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _check_dev("final_state", final_state, torch.float32)
    if initial_state is not None:
        _check_dev("initial_state", initial_state, torch.float32)
        if tuple(initial_state.shape) != (B, H, dk, dv):
            raise ValueError("initial_state must be [B,H,dk,dv]")
    g = _gamma_array(gamma, H)
    dt = _dtype_code(q)
    ws, nws = _workspace(lib.retention_fwd_workspace_bytes(B, H, T, dk, dv, int(chunk), dt), q.device,
                         workspace)
    if initial_state is None:
        rc = lib.retention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk), out.data_ptr(),
                               _ptr(final_state), B, H, T, dk, dv, dt, _ptr(ws), nws, _stream(q))
    else:
        rc = lib.retention_fwd_from_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk),
                                          initial_state.data_ptr(), out.data_ptr(), _ptr(final_state),
                                          B, H, T, dk, dv, dt, _ptr(ws), nws, _stream(q))
    _raise(rc)
    return out, final_state


def retention_fwd_noalloc(q, k, v, gamma, chunk: int = 64, out=None, final_state=None, want_state: bool = True):
    """retention_fwd without a workspace: the library keeps the segment states
    in its own device array (RET_NOALLOC_MAX_WORKSPACE bytes per GPU), so the
    C call allocates nothing.  Pass `out` (and `final_state`) to keep this
    wrapper from allocating them.  Calls that overlap in time on one GPU race."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    if final_state is None and want_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _check_dev("final_state", final_state, torch.float32)
    g = _gamma_array(gamma, H)
    rc = lib.retention_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk), out.data_ptr(),
                                   _ptr(final_state), B, H, T, dk, dv, _dtype_code(q), _stream(q))
    _raise(rc)
    return out, final_state


def retention_fwd_normalized(q, k, v, gamma, norm: str = "group", eps: float = 1e-5, chunk: int = 64, out=None,
                             workspace=None):
    """Retention divided by its score row sum floored at 1 (norm="rowsum"),
    then GroupNorm over each row (norm="group"), fused into the walk.

    bf16 or float32 (float32 GroupNorm is fused where one workgroup holds whole rows,
    else a second in-place pass over out).
    q, k: [B,H,T,dk]; v: [B,H,T,dv].  Returns out [B,H,T,dv]."""
    lib = load_library()
    codes = {"rowsum": RET_NORM_ROWSUM, "group": RET_NORM_GROUP}
    if norm not in codes:
        raise ValueError("norm must be 'rowsum' or 'group'")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    g = _gamma_array(gamma, H)
    dt = _dtype_code(q)
    ws, nws = _workspace(lib.retention_fwd_normalized_workspace_bytes(B, H, T, dk, dv, int(chunk), dt), q.device,
                         workspace)
    rc = lib.retention_fwd_normalized(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk), codes[norm],
                                      float(eps), out.data_ptr(), B, H, T, dk, dv, dt, _ptr(ws), nws, _stream(q))
    _raise(rc)
    return out


def gla_fwd(q, k, v, log_gate, out=None, final_state=None, want_state: bool = True, workspace=None):
    """Gated linear attention with per-token, per-key-channel gates
    exp(log_gate): q, k [B,H,T,dk] and v [B,H,T,dv] in float32 or bfloat16
    (one dtype), log_gate [B,H,T,dk] float32, on the GPU.  Returns
    (out [B,H,T,dv] in the input dtype, final_state [B,H,dk,dv] float32 or None)."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    _check_dev("log_gate", log_gate, torch.float32)
    if q.dim() != 4 or k.shape != q.shape or log_gate.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k, log_gate must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    if final_state is None and want_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _check_dev("final_state", final_state, torch.float32)
    dt = _dtype_code(q)
    ws, nws = _workspace(lib.gla_fwd_workspace_bytes(B, H, T, dk, dv, dt), q.device, workspace)
    rc = lib.gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gate.data_ptr(), out.data_ptr(),
                     _ptr(final_state), B, H, T, dk, dv, dt, _ptr(ws), nws, _stream(q))
    _raise(rc)
    return out, final_state


def retention_bwd(q, k, v, gamma, dout, chunk: int = 64, dq=None, dk=None, dv=None, workspace=None,
                  fwd_workspace=None):
    """Gradients (dq, dk, dv) of retention_fwd (zero initial state) given
    dout = dL/dout; all tensors [B,H,T,*] in one dtype on the GPU.

    fwd_workspace: optional uint8 GPU tensor that a retention_fwd call on the
    same k, v, gamma and chunk was given as its workspace (and that nothing has
    written since); dq then reuses the segment states it holds.  It must not be
    the workspace of this call."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3] or dout.shape != v.shape:
        raise ValueError("q, k must be [B,H,T,dk] and v, dout [B,H,T,dv]")
    B, H, T, d_k = q.shape
    d_v = v.shape[3]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_dev(n, t, q.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    g = _gamma_array(gamma, H)
    dt = _dtype_code(q)
    ws, nws = _workspace(lib.retention_bwd_workspace_bytes(B, H, T, d_k, d_v, int(chunk), dt), q.device, workspace)
    if fwd_workspace is None:
        rc = lib.retention_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk), dout.data_ptr(),
                               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, d_k, d_v, dt, _ptr(ws), nws,
                               _stream(q))
    else:
        _check_dev("fwd_workspace", fwd_workspace, torch.uint8)
        rc = lib.retention_bwd_from_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, int(chunk), dout.data_ptr(),
                                        _ptr(fwd_workspace), fwd_workspace.numel(), dq.data_ptr(), dk.data_ptr(),
                                        dv.data_ptr(), B, H, T, d_k, d_v, dt, _ptr(ws), nws, _stream(q))
    _raise(rc)
    return dq, dk, dv


class _Retention(torch.autograd.Function):
    """Autograd glue: forward is retention_fwd, backward is retention_bwd_from_fwd
    with the forward's workspace (its segment states), kept until backward."""

    @staticmethod
    def forward(ctx, q, k, v, gamma, chunk):
        B, H, T, d_k = q.shape
        n = retention_fwd_workspace_bytes(B, H, T, d_k, v.shape[3], chunk, q.dtype)
        fws = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
        out, _ = retention_fwd(q, k, v, gamma, chunk=chunk, want_state=False, workspace=fws)
        ctx.save_for_backward(q, k, v)
        ctx.gamma, ctx.chunk, ctx.fws = gamma, chunk, fws
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v = ctx.saved_tensors
        # without a forward workspace (one segment, or the fp32 path) there are no states to share
        dq, dk, dv = retention_bwd(q, k, v, ctx.gamma, dout.contiguous(), chunk=ctx.chunk, fwd_workspace=ctx.fws)
        ctx.fws = None
        return dq, dk, dv, None, None


def retention(q, k, v, gamma, chunk: int = 64):
    """Differentiable chunkwise retention (zero initial state): out [B,H,T,dv].

    gamma is a host list / array of H decays (not differentiated)."""
    g = gamma.detach().cpu().tolist() if isinstance(gamma, torch.Tensor) else gamma
    return _Retention.apply(q, k, v, g, int(chunk))


def retention_decode_step(q, k, v, gamma, state, out=None):
    """One recurrent step S <- gamma S + k v^T, out = q S, state updated in place.

    q, k: [N,H,dk]; v: [N,H,dv] (float32 or bfloat16); state: [N,H,dk,dv]
    float32.  Returns out [N,H,dv] in the input dtype.
    """
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    _check_dev("state", state, torch.float32)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[2]
    if tuple(state.shape) != (N, H, dk, dv):
        raise ValueError("state must be [N,H,dk,dv]")
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    g = _gamma_array(gamma, H)
    rc = lib.retention_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, state.data_ptr(),
                                   out.data_ptr(), N, H, dk, dv, _dtype_code(q), _stream(q))
    _raise(rc)
    return out


def linear_attn_fwd(q, k, v, phi: str = "elu1", eps: float = 1e-6, out=None, workspace=None,
                    initial_state=None, return_state: bool = False, final_state=None):
    """Causal linear attention with phi = elu+1 and its normaliser.

    q, k: [B,H,T,dk]; v: [B,H,T,dv].  Returns out [B,H,T,dv], or
    (out, S, z) when return_state is True or final_state = (S, z) buffers are
    passed (S [B,H,dk,dv], z [B,H,dk], float32).  initial_state: optional
    (S0, z0) pair after earlier tokens (either may be None for zero).
    workspace: optional uint8 GPU tensor of at least
    linear_attn_workspace_bytes(...) bytes; one is allocated per call when it
    is omitted.
    """
    lib = load_library()
    if phi not in ("elu1", RET_PHI_ELU1):
        raise ValueError("phi must be 'elu1'")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    dt = _dtype_code(q)
    ws, nws = _workspace(lib.linear_attn_workspace_bytes(B, H, T, dk, dv, dt), q.device, workspace)
    S0 = z0 = None
    if initial_state is not None:
        S0, z0 = initial_state
    fS = fz = None
    if final_state is not None:
        fS, fz = final_state
    elif return_state:
        fS = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
        fz = torch.empty((B, H, dk), dtype=torch.float32, device=q.device)
    for name, t, shp in (("initial S", S0, (B, H, dk, dv)), ("initial z", z0, (B, H, dk)),
                         ("final S", fS, (B, H, dk, dv)), ("final z", fz, (B, H, dk))):
        if t is not None:
            _check_dev(name, t, torch.float32)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must be {list(shp)}")
    if S0 is None and z0 is None and fS is None and fz is None:
        rc = lib.linear_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), RET_PHI_ELU1, out.data_ptr(),
                                 B, H, T, dk, dv, dt, float(eps), _ptr(ws), nws, _stream(q))
        _raise(rc)
        return out
    rc = lib.linear_attn_fwd_from_state(q.data_ptr(), k.data_ptr(), v.data_ptr(), RET_PHI_ELU1, _ptr(S0),
                                        _ptr(z0), out.data_ptr(), _ptr(fS), _ptr(fz), B, H, T, dk, dv, dt,
                                        float(eps), _ptr(ws), nws, _stream(q))
    _raise(rc)
    if fS is None and fz is None:
        return out
    return out, fS, fz


def linear_attn_decode_step(q, k, v, S, z, eps: float = 1e-6, out=None, phi: str = "elu1"):
    """One decode step of causal linear attention (phi = elu+1), in place:
    S <- S + phi(k) v^T, z <- z + phi(k), out = S^T phi(q) / (z^T phi(q) + eps).

    q, k: [N,H,dk]; v: [N,H,dv] (float32 or bfloat16); S: [N,H,dk,dv] and
    z: [N,H,dk] float32.  Returns out [N,H,dv] in the input dtype.
    """
    lib = load_library()
    if phi not in ("elu1", RET_PHI_ELU1):
        raise ValueError("phi must be 'elu1'")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(n, t, q.dtype)
    _check_dev("S", S, torch.float32)
    _check_dev("z", z, torch.float32)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[2]
    if tuple(S.shape) != (N, H, dk, dv) or tuple(z.shape) != (N, H, dk):
        raise ValueError("S must be [N,H,dk,dv] and z [N,H,dk]")
    if out is None:
        out = torch.empty_like(v)
    _check_dev("out", out, v.dtype)
    rc = lib.linear_attn_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), RET_PHI_ELU1, S.data_ptr(),
                                     z.data_ptr(), out.data_ptr(), N, H, dk, dv, _dtype_code(q), float(eps),
                                     _stream(q))
    _raise(rc)
    return out
