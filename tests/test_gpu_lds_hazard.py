"""LDS hazard self-check (GPU): the -DRET_DEBUG build overwrites every LDS
buffer with NaN words as soon as the barrier protocol says no wave reads it
any more (the chunk tiles of the segment walks, the fused backward walk and
the gated walk; the block ring of the state kernel).  A read that a missing or
misplaced barrier let through would then see NaN instead of stale data, so
the debug build's outputs must equal the normal build's bit for bit, and
contain no NaN, on shapes that take every walk through several chunks per
segment, several segments, ragged tails and (for the gated walk) both the
fast and the exact path.  Both builds are called through the C ABI on the
same inputs."""
import ctypes

import numpy as np
import pytest
import torch

import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbg():
    lib = rc.load_debug_library()
    yield lib
    lib.retention_set_plan_override(0, 0, 0, 0)


def _both(dbg, segments):
    """The same segment count in both builds (each library keeps its own
    per-thread plan override)."""
    rc.set_plan_override(segments=segments)
    assert dbg.retention_set_plan_override(0, int(segments or 0), 0, 0) == 0


def _bf16(seed, shape, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).cuda()


def _ws(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")


def _same(tag, a, b):
    torch.cuda.synchronize()
    assert not torch.isnan(b.float()).any(), f"{tag}: the debug build produced NaN (an LDS hazard)"
    assert torch.equal(a, b), f"{tag}: debug build differs from the normal build"


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _gam(H):
    g = wl.gammas("msr_spread", H)
    return (ctypes.c_float * H)(*np.asarray(g, dtype=np.float32).tolist())


@pytest.mark.parametrize("chunk,dk,dv,T,G", [(128, 128, 128, 1500, 3), (64, 64, 128, 1000, 4), (128, 64, 64, 700, 1)])
def test_forward_walk_and_state_kernel(dbg, plan, chunk, dk, dv, T, G):
    B, H = 1, 3
    q, k, v = _bf16(1, (B, H, T, dk), dk ** -0.5), _bf16(2, (B, H, T, dk)), _bf16(3, (B, H, T, dv))
    _both(dbg, G)
    gam = wl.gammas("msr_spread", H)
    ref, ref_s = rc.retention_fwd(q, k, v, gam, chunk=chunk)
    out, fs = torch.empty_like(ref), torch.empty_like(ref_s)
    ws = _ws(dbg.retention_fwd_workspace_bytes(B, H, T, dk, dv, chunk, rc.RET_BF16))
    assert dbg.retention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _gam(H), chunk, out.data_ptr(), fs.data_ptr(),
                             B, H, T, dk, dv, rc.RET_BF16, ws.data_ptr(), ws.numel(), _stream()) == 0
    _same(f"retention_fwd C={chunk} d={dk}/{dv} G={G} out", ref, out)
    _same("final state", ref_s, fs)


@pytest.mark.parametrize("dk,T,G", [(64, 1500, 3), (128, 900, 2)])
def test_linear_attention_walk(dbg, plan, dk, T, G):
    B, H, dv = 2, 2, 64
    q, k, v = _bf16(4, (B, H, T, dk), 0.5), _bf16(5, (B, H, T, dk), 0.5), _bf16(6, (B, H, T, dv))
    _both(dbg, G)
    ref = rc.linear_attn_fwd(q, k, v)
    out = torch.empty_like(ref)
    ws = _ws(dbg.linear_attn_workspace_bytes(B, H, T, dk, dv, rc.RET_BF16))
    assert dbg.linear_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), rc.RET_PHI_ELU1, out.data_ptr(), B, H, T, dk,
                               dv, rc.RET_BF16, ctypes.c_float(1e-6), ws.data_ptr(), ws.numel(), _stream()) == 0
    _same(f"linear_attn_fwd dk={dk} G={G}", ref, out)


@pytest.mark.parametrize("norm", ["rowsum", "group"])
def test_normalised_walk(dbg, plan, norm):
    B, H, T, d = 1, 2, 1100, 128
    q, k, v = _bf16(7, (B, H, T, d), d ** -0.5), _bf16(8, (B, H, T, d)), _bf16(9, (B, H, T, d))
    _both(dbg, 3)
    gam = wl.gammas("msr_spread", H)
    ref = rc.retention_fwd_normalized(q, k, v, gam, chunk=128, norm=norm)
    out = torch.empty_like(ref)
    code = rc.RET_NORM_ROWSUM if norm == "rowsum" else rc.RET_NORM_GROUP
    ws = _ws(dbg.retention_fwd_normalized_workspace_bytes(B, H, T, d, d, 128, rc.RET_BF16))
    assert dbg.retention_fwd_normalized(q.data_ptr(), k.data_ptr(), v.data_ptr(), _gam(H), 128, code,
                                        ctypes.c_float(1e-5), out.data_ptr(), B, H, T, d, d, rc.RET_BF16, ws.data_ptr(),
                                        ws.numel(), _stream()) == 0
    _same(f"retention_fwd_normalized {norm}", ref, out)


@pytest.mark.parametrize("dk,dv,T,G", [(128, 128, 1300, 3), (64, 128, 700, 2)])
def test_fused_backward_walk(dbg, plan, dk, dv, T, G):
    B, H = 1, 2
    q, k, v = _bf16(10, (B, H, T, dk), dk ** -0.5), _bf16(11, (B, H, T, dk)), _bf16(12, (B, H, T, dv))
    dout = _bf16(13, (B, H, T, dv))
    _both(dbg, G)
    gam = wl.gammas("msr_spread", H)
    rq, rk, rv = rc.retention_bwd(q, k, v, gam, dout, chunk=128)
    dq, dk_, dv_ = torch.empty_like(rq), torch.empty_like(rk), torch.empty_like(rv)
    ws = _ws(dbg.retention_bwd_workspace_bytes(B, H, T, dk, dv, 128, rc.RET_BF16))
    assert dbg.retention_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _gam(H), 128, dout.data_ptr(), dq.data_ptr(),
                             dk_.data_ptr(), dv_.data_ptr(), B, H, T, dk, dv, rc.RET_BF16, ws.data_ptr(), ws.numel(),
                             _stream()) == 0
    _same(f"retention_bwd d={dk}/{dv} G={G} dq", rq, dq)
    _same("dk", rk, dk_)
    _same("dv", rv, dv_)


@pytest.mark.parametrize("dk,dtype", [(64, torch.float32), (128, torch.float32), (64, torch.bfloat16)])
def test_gated_walk(dbg, plan, dk, dtype):
    """Two buffer sets at dk = 64, one at dk = 128; one chunk on the exact path."""
    B, H, T, dv = 1, 2, 700, 64
    g = torch.Generator().manual_seed(14)
    q = (torch.randn((B, H, T, dk), generator=g) / 8).to(dtype).cuda()
    k = (torch.randn((B, H, T, dk), generator=g) / 8).to(dtype).cuda()
    v = torch.randn((B, H, T, dv), generator=g).to(dtype).cuda()
    lg = torch.nn.functional.logsigmoid(torch.randn((B, H, T, dk), generator=g) + 2.0)
    lg[:, :, 128:192] = torch.nn.functional.logsigmoid(torch.randn((B, H, 64, dk), generator=g) - 3.0) * 8
    lg = lg.cuda()
    _both(dbg, 3)
    ref, ref_s = rc.gla_fwd(q, k, v, lg)
    out, fs = torch.empty_like(ref), torch.empty_like(ref_s)
    dt = rc.RET_F32 if dtype == torch.float32 else rc.RET_BF16
    ws = _ws(dbg.gla_fwd_workspace_bytes(B, H, T, dk, dv, dt))
    assert dbg.gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), lg.data_ptr(), out.data_ptr(), fs.data_ptr(), B, H, T,
                       dk, dv, dt, ws.data_ptr(), ws.numel(), _stream()) == 0
    _same(f"gla_fwd dk={dk} {dtype} out", ref, out)
    _same("final state", ref_s, fs)
