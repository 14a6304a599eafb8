"""fp64 CPU oracle for causal retention and causal linear attention.

TEST INFRASTRUCTURE ONLY.  This package is the checker for the HIP path.  Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the library under test never does, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double), built with gcc
into ``liboracle.so`` next to it.  This module only marshals numpy arrays.
Each wrapper names the passage its C function follows; see ``oracle.c`` for
the citations in full.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (worked examples printed on the pages, closed
forms, the gamma = 1 and associativity identities, brute force on tiny
inputs).  Values that no page prints (bf16 inputs, long decode runs, ragged
tails) are covered by the same code paths; the pins fix the arithmetic, not
those particular numbers.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ELU1_EPS = 1e-6  # the denominator guard the pages add "as written"


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` with gcc -O2 -fopenmp into a shared library."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_D = ctypes.POINTER(ctypes.c_double)
_L = ctypes.POINTER(ctypes.c_long)
_l = ctypes.c_long


def load(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every wrapper through another build of oracle.c.

    The mutation tests use this to run the pins against deliberately broken
    copies of the oracle and show that each copy fails at least one pin.
    """
    global _lib
    with _lock:
        old = _lib
        _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        with _lock:
            _lib = old


def _bind(lib):
    lib.oracle_retention_recurrent.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l,
                                               _D, _D, _D, ctypes.c_int]
    lib.oracle_retention_parallel.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D]
    lib.oracle_retention_rows.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l, _L, _l,
                                          _D, ctypes.c_int]
    lib.oracle_retention_chunkwise.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l, _l,
                                               _D, _D]
    lib.oracle_decode_steps.argtypes = [_D, _D, _D, _D, _D, _D, _l, _l, _l, _l, _l,
                                        ctypes.c_int]
    lib.oracle_linattn_recurrent.argtypes = [_D, _D, _D, ctypes.c_double, _l, _l, _l,
                                             _l, _l, _D, _D, _D, _D, _D, ctypes.c_int]
    lib.oracle_linattn_decode_steps.argtypes = [_D, _D, _D, ctypes.c_double, _D, _D, _D,
                                                _l, _l, _l, _l, _l, ctypes.c_int]
    lib.oracle_linattn_parallel.argtypes = [_D, _D, _D, ctypes.c_double, _l, _l, _l,
                                            _l, _l, _D]
    lib.oracle_linattn_rows.argtypes = [_D, _D, _D, ctypes.c_double, _l, _l, _l, _l, _l,
                                        _L, _l, _D, ctypes.c_int]
    lib.oracle_retention_bwd.argtypes = [_D, _D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, _D,
                                         ctypes.c_int]
    lib.oracle_retention_normalized.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l, ctypes.c_int,
                                                ctypes.c_double, _D, ctypes.c_int]
    lib.oracle_gla_recurrent.argtypes = [_D, _D, _D, _D, _l, _l, _l, _l, _l, _D, _D, ctypes.c_int]
    lib.oracle_threads_used.argtypes = [ctypes.c_int]
    for name in ("oracle_retention_recurrent", "oracle_retention_parallel",
                 "oracle_retention_rows", "oracle_retention_chunkwise",
                 "oracle_decode_steps", "oracle_linattn_recurrent",
                 "oracle_linattn_decode_steps", "oracle_retention_bwd",
                 "oracle_retention_normalized", "oracle_gla_recurrent",
                 "oracle_linattn_parallel", "oracle_linattn_rows",
                 "oracle_threads_used"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    """Any array-like (numpy, torch CPU tensor) -> C-contiguous float64."""
    if hasattr(x, "detach"):  # torch tensor: widen exactly, on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def _shape4(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, T, dk = q.shape
    if k.shape != (B, H, T, dk) or v.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v")
    return B, H, T, dk, v.shape[3]


def threads_used(nthreads: int) -> int:
    return int(load().oracle_threads_used(int(nthreads)))


def retention_recurrent(q, k, v, gamma, init_state=None, nthreads: int = 1):
    """Retention, recurrent form (RetNet page, "Recurrent Representation").

    Returns (out [B,H,T,dv], final_state [B,H,dk,dv]) in float64.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    B, H, T, dk, dv = _shape4(q, k, v)
    if g.shape != (H,):
        raise ValueError("gamma must have H entries")
    out = np.zeros((B, H, T, dv))
    fs = np.zeros((B, H, dk, dv))
    init = None
    if init_state is not None:
        init = _f64(init_state)
        if init.shape != (B, H, dk, dv):
            raise ValueError("init_state must be [B,H,dk,dv]")
    lib = load()
    _check(lib.oracle_retention_recurrent(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv,
                                          _p(init) if init is not None else None,
                                          _p(out), _p(fs), int(nthreads)),
           "oracle_retention_recurrent")
    return out, fs


def retention_parallel(q, k, v, gamma):
    """Retention, parallel form O = (QK^T (.) D) V, brute force (tiny T)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    B, H, T, dk, dv = _shape4(q, k, v)
    out = np.zeros((B, H, T, dv))
    _check(load().oracle_retention_parallel(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv,
                                            _p(out)), "oracle_retention_parallel")
    return out


def retention_rows(q, k, v, gamma, rows, nthreads: int = 1):
    """Rows (b, h, t) of the retention output from the parallel definition."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    B, H, T, dk, dv = _shape4(q, k, v)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    out = np.zeros((r.shape[0], dv))
    _check(load().oracle_retention_rows(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv,
                                        r.ctypes.data_as(_L), r.shape[0], _p(out),
                                        int(nthreads)), "oracle_retention_rows")
    return out


def retention_chunkwise(q, k, v, gamma, chunk: int):
    """The chunk equations derived from the recurrence, in fp64."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    B, H, T, dk, dv = _shape4(q, k, v)
    out = np.zeros((B, H, T, dv))
    fs = np.zeros((B, H, dk, dv))
    _check(load().oracle_retention_chunkwise(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv,
                                             int(chunk), _p(out), _p(fs)),
           "oracle_retention_chunkwise")
    return out, fs


def decode_steps(q, k, v, gamma, state, nsteps: int = 1, nthreads: int = 1):
    """nsteps recurrent decode steps with the same token (q, k, v).

    q, k: [N,H,dk]; v: [N,H,dv]; state: [N,H,dk,dv].  Returns
    (out [N,H,dv] of the last step, new_state) -- the input state is not
    modified.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    S = _f64(state).copy()
    if q.ndim != 3:
        raise ValueError("q must be [N,H,dk]")
    N, H, dk = q.shape
    dv = v.shape[2]
    if S.shape != (N, H, dk, dv):
        raise ValueError("state must be [N,H,dk,dv]")
    out = np.zeros((N, H, dv))
    _check(load().oracle_decode_steps(_p(q), _p(k), _p(v), _p(g), _p(S), _p(out), N, H,
                                      dk, dv, int(nsteps), int(nthreads)),
           "oracle_decode_steps")
    return out, S


def gla_recurrent(q, k, v, log_gate, nthreads: int = 1):
    """Gated linear attention with per-token, per-key-channel gates
    exp(log_gate) ("Efficient and Sparse Transformers", section "Gated Linear
    Attention"), recurrent form.  Returns (out [B,H,T,dv], final S [B,H,dk,dv])."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(log_gate)
    B, H, T, dk, dv = _shape4(q, k, v)
    if g.shape != (B, H, T, dk):
        raise ValueError("log_gate must be [B,H,T,dk]")
    out = np.zeros((B, H, T, dv))
    fs = np.zeros((B, H, dk, dv))
    _check(load().oracle_gla_recurrent(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv, _p(out), _p(fs),
                                       int(nthreads)), "oracle_gla_recurrent")
    return out, fs


GROUPNORM_EPS = 1e-5


def retention_normalized(q, k, v, gamma, group: bool = False, eps: float = GROUPNORM_EPS, nthreads: int = 1):
    """Retention divided by its decayed score row sum floored at 1 in size,
    optionally followed by GroupNorm over each row ("Linear attention" page,
    box "An LSTM whose cell is linear attention"; "RetNet", the layer's
    optional GroupNorm).  Returns out [B,H,T,dv]."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1)
    B, H, T, dk, dv = _shape4(q, k, v)
    if g.shape != (H,):
        raise ValueError("gamma must have H entries")
    out = np.zeros((B, H, T, dv))
    _check(load().oracle_retention_normalized(_p(q), _p(k), _p(v), _p(g), B, H, T, dk, dv,
                                              1 if group else 0, float(eps), _p(out), int(nthreads)),
           "oracle_retention_normalized")
    return out


def retention_bwd(q, k, v, gamma, dout, nthreads: int = 1):
    """Gradients (dq, dk, dv) of retention from a zero state, given dout,
    as cumulative sums forward (queries) and backward (keys, values) in time
    ("Linear attention" page, "Decoding, training, and what each costs")."""
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(gamma).reshape(-1), _f64(dout)
    B, H, T, dk, dv = _shape4(q, k, v)
    if do.shape != (B, H, T, dv):
        raise ValueError("dout must be [B,H,T,dv]")
    if g.shape != (H,):
        raise ValueError("gamma must have H entries")
    dq = np.zeros((B, H, T, dk))
    dkk = np.zeros((B, H, T, dk))
    dvv = np.zeros((B, H, T, dv))
    _check(load().oracle_retention_bwd(_p(q), _p(k), _p(v), _p(g), _p(do), B, H, T, dk, dv,
                                       _p(dq), _p(dkk), _p(dvv), int(nthreads)),
           "oracle_retention_bwd")
    return dq, dkk, dvv


def linattn_recurrent(q, k, v, eps: float = ELU1_EPS, init_S=None, init_z=None,
                      nthreads: int = 1):
    """Causal linear attention, phi = elu+1 with normaliser, recurrent form
    ("Linear attention" page, recurrent-form box), from (init_S, init_z)
    (zero when None).

    Returns (out [B,H,T,dv], S [B,H,dk,dv], z [B,H,dk]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk, dv = _shape4(q, k, v)
    out = np.zeros((B, H, T, dv))
    S = np.zeros((B, H, dk, dv))
    z = np.zeros((B, H, dk))
    iS = iz = None
    if init_S is not None:
        iS = _f64(init_S)
        if iS.shape != (B, H, dk, dv):
            raise ValueError("init_S must be [B,H,dk,dv]")
    if init_z is not None:
        iz = _f64(init_z)
        if iz.shape != (B, H, dk):
            raise ValueError("init_z must be [B,H,dk]")
    _check(load().oracle_linattn_recurrent(_p(q), _p(k), _p(v), float(eps), B, H, T, dk,
                                           dv, _p(iS) if iS is not None else None,
                                           _p(iz) if iz is not None else None,
                                           _p(out), _p(S), _p(z), int(nthreads)),
           "oracle_linattn_recurrent")
    return out, S, z


def linattn_decode_steps(q, k, v, S, z, eps: float = ELU1_EPS, nsteps: int = 1,
                         nthreads: int = 1):
    """nsteps decode steps of causal linear attention with the same token
    ("Linear attention" page, the decode-step exercise).

    q, k: [N,H,dk]; v: [N,H,dv]; S: [N,H,dk,dv]; z: [N,H,dk].  Returns
    (out [N,H,dv] of the last step, S_new, z_new); the inputs are not
    modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(S).copy()
    z = _f64(z).copy()
    if q.ndim != 3:
        raise ValueError("q must be [N,H,dk]")
    N, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != q.shape or v.shape[:2] != (N, H):
        raise ValueError("shape mismatch between q, k, v")
    if S.shape != (N, H, dk, dv) or z.shape != (N, H, dk):
        raise ValueError("S must be [N,H,dk,dv] and z [N,H,dk]")
    out = np.zeros((N, H, dv))
    _check(load().oracle_linattn_decode_steps(_p(q), _p(k), _p(v), float(eps), _p(S), _p(z),
                                              _p(out), N, H, dk, dv, int(nsteps),
                                              int(nthreads)),
           "oracle_linattn_decode_steps")
    return out, S, z


def linattn_parallel(q, k, v, eps: float = ELU1_EPS):
    """Causal linear attention, masked parallel form, brute force (tiny T)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk, dv = _shape4(q, k, v)
    out = np.zeros((B, H, T, dv))
    _check(load().oracle_linattn_parallel(_p(q), _p(k), _p(v), float(eps), B, H, T, dk,
                                          dv, _p(out)), "oracle_linattn_parallel")
    return out


def linattn_rows(q, k, v, rows, eps: float = ELU1_EPS, nthreads: int = 1):
    """Rows (b, h, t) of the linear-attention output from the parallel form."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk, dv = _shape4(q, k, v)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    out = np.zeros((r.shape[0], dv))
    _check(load().oracle_linattn_rows(_p(q), _p(k), _p(v), float(eps), B, H, T, dk, dv,
                                      r.ctypes.data_as(_L), r.shape[0], _p(out),
                                      int(nthreads)), "oracle_linattn_rows")
    return out


def frobenius_parts(x, ref) -> tuple[float, float]:
    """(||x - ref||_F, ||ref||_F) in float64: the numerator and denominator of
    the relative Frobenius error, kept apart so that the errors of pieces of a
    tensor (head groups compared one after another) combine exactly."""
    x = _f64(x)
    ref = _f64(ref)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch: {x.shape} vs {ref.shape}")
    return float(np.linalg.norm((x - ref).ravel())), float(np.linalg.norm(ref.ravel()))


def _ratio(num: float, den: float) -> float:
    # a zero reference has no relative error: the absolute one is reported, so
    # only an x that is zero as well passes a small tolerance
    return num / den if den > 0.0 else num


def rel_frobenius(x, ref) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F (float64), measured
    against the reference; ||x - ref||_F itself when ref is all zeros."""
    return _ratio(*frobenius_parts(x, ref))


def combine_rel_frobenius(parts) -> float:
    """The relative Frobenius error of a whole tensor from the
    frobenius_parts of disjoint pieces that cover it."""
    num2 = sum(n * n for n, _ in parts)
    den2 = sum(d * d for _, d in parts)
    return _ratio(float(np.sqrt(num2)), float(np.sqrt(den2)))


def rel_frobenius_per_slice(x, ref, lead: int = 2) -> np.ndarray:
    """Relative Frobenius error of every slice over the first `lead` axes
    (per (b, h) for [B, H, ...] tensors), as an array of that shape."""
    x = _f64(x)
    ref = _f64(ref)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch: {x.shape} vs {ref.shape}")
    shp = x.shape[:lead]
    d = (x - ref).reshape(shp + (-1,))
    r = ref.reshape(shp + (-1,))
    num = np.sqrt(np.sum(d * d, axis=-1))
    den = np.sqrt(np.sum(r * r, axis=-1))
    return np.where(den > 0.0, num / np.where(den > 0.0, den, 1.0), num)
