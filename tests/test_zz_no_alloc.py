"""retention_fwd_noalloc through the C ABI against retention_fwd (needs a
gfx950 GPU).

The allocation-free variant keeps the segment states in the library's own
device array instead of a caller workspace.  It runs the same kernels with
the same plan, so its outputs must equal retention_fwd's bit for bit; both are
also held to the oracle.  Two calls in a row, the second smaller (fewer
segments, another shape), show that whatever the first call left in the
shared array does not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

RET_ERR_WORKSPACE = -9


def _noalloc(lib, q, k, v, gamma, chunk, out, fs):
    B, H, T, dk = q.shape
    dv = v.shape[3]
    g = (ctypes.c_float * H)(*np.asarray(gamma, dtype=np.float32).tolist())
    dt = 1 if q.dtype == torch.bfloat16 else 0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.retention_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, chunk, out.data_ptr(),
                                     fs.data_ptr() if fs is not None else None, B, H, T, dk, dv, dt, stream)


def _case(lib, name, seed, chunk, heads_checked, **over):
    w = wl.WORKLOADS[name].with_(**over) if over else wl.WORKLOADS[name]
    inp = wl.make_inputs(w, seed)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    B, H, T, dk = q.shape
    need = rc.retention_fwd_workspace_bytes(B, H, T, dk, v.shape[3], chunk, q.dtype)
    print(f"[noalloc] {name} {tuple(q.shape)} dv={v.shape[3]} chunk={chunk}: segment states {need} bytes", flush=True)
    out = torch.full_like(v, float("nan"))
    fs = torch.full((B, H, dk, v.shape[3]), float("nan"), dtype=torch.float32, device="cuda")
    assert _noalloc(lib, q, k, v, inp["gamma"], chunk, out, fs) == 0, rc.last_error()
    ref_out, ref_fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(fs, ref_fs), "noalloc differs from retention_fwd"
    tol = 2e-2 if q.dtype == torch.bfloat16 else 1e-4
    sl = slice(0, heads_checked)
    ro, rs = oracle.retention_recurrent(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], inp["gamma"][sl],
                                        nthreads=16)
    parity.check(f"noalloc {name} out (heads 0..{heads_checked - 1})", out[:, sl].float().cpu().numpy(), ro, tol)
    parity.check(f"noalloc {name} final_state", fs[:, sl].cpu().numpy(), rs, tol)
    return need


def test_noalloc_matches_retention_fwd_on_two_calls_in_a_row():
    lib = rc.load_library()
    # first: the [1, 32, 65536, 128] bf16 forward (8 segments per head, 14.7 MB of states)
    big = _case(lib, "ret_fwd_long_bf16", 0, 128, 8)
    # second, smaller: fewer heads, a ragged length, other widths and chunk
    small = _case(lib, "ret_fwd_long_bf16", 1, 64, 3, B=2, H=3, T=5000, dk=64, dv=128)
    assert 0 < small < big
    # fp32 (value-slice path with its own segment layout), then bf16 again with one segment
    _case(lib, "ret_fwd_mh_f32", 2, 64, 8)
    _case(lib, "ret_fwd_long_bf16", 3, 128, 2, H=2, T=300)


def test_noalloc_rejects_sizes_beyond_its_array():
    lib = rc.load_library()
    q = torch.zeros((1, 64, 65536, 128), dtype=torch.bfloat16, device="cuda")
    with rc.plan_override(segments=16):
        need = rc.retention_fwd_workspace_bytes(1, 64, 65536, 128, 128, 128, torch.bfloat16)
        assert need > (32 << 20)
        out = torch.empty_like(q)
        assert _noalloc(lib, q, q, q, [0.9] * 64, 128, out, None) == RET_ERR_WORKSPACE
        msg = rc.last_error()  # read before the override is reset (a successful call clears it)
    assert "retention_fwd_noalloc" in msg and "retention_fwd with a workspace" in msg
