"""Retention gradients (retention_bwd) against the fp64 oracle (needs a gfx950 GPU).

retention_bwd returns dq, dk, dv of retention_fwd from a zero state, given
dout.  The library computes them as three chunkwise walks (dq forward in
time, dk and dv over the time-reversed sequence); the oracle computes them as
cumulative sums forward and backward in time.  Cases: bf16 (segment path,
several forced segment counts) and fp32 (value-slice path), chunks 64 and
128, every (dk, dv) pair, ragged and short lengths, unit and small decays, the
full long-sequence shape on two heads, and the autograd wrapper.  The same
for retention_bwd_from_fwd, whose dq walk reads the segment states that the
forward left in its workspace (transposed) instead of summing them again.
Tolerances: relative Frobenius error 1e-4 (fp32), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _inputs(seed, dtype, B, H, T, dk, dv, chunk=64):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(B=B, H=H, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype,
                                              scale=1.0 / np.sqrt(dk))
    inp = wl.make_inputs(w, seed)
    g = torch.Generator().manual_seed(seed + 500)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inp["do"] = torch.randn((B, H, T, dv), generator=g).to(tdt)
    return w, inp


def _segments(plan, G):
    plan(segments=G)


def _check(tag, got, ref, tol):
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        parity.check(f"{tag} {name}", x, r, tol)


def _run(inp, chunk):
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    dq, dk, dv = rc.retention_bwd(q, k, v, inp["gamma"], do, chunk=chunk)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)]


@pytest.mark.parametrize("dtype,G", [("f32", None), ("f32", 3), ("bf16", None), ("bf16", 1), ("bf16", 5)])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 1000), (64, 128, 129), (128, 64, 700)])
def test_bwd_small_full(dtype, G, chunk, dk, dv, T, plan):
    w, inp = _inputs(51, dtype, 2, 3, T, dk, dv, chunk)
    _segments(plan, G)
    print(f"[bwd] {dtype} G={G} C={chunk} dk={dk} dv={dv} T={T}", flush=True)
    got = _run(inp, chunk)
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"], nthreads=8)
    _check(f"bwd {dtype} G={G} C={chunk} dk={dk} dv={dv} T={T}", got, ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 127, 128, 129])
def test_bwd_short_and_ragged(dtype, T, plan):
    w, inp = _inputs(52, dtype, 1, 2, T, 64, 64)
    _segments(plan, 2)
    got = _run(inp, 64)
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"])
    _check(f"bwd short {dtype} T={T}", got, ref, TOL[dtype])


def test_bwd_zero_length_and_empty_batch():
    q = torch.zeros((1, 2, 0, 64), device="cuda", dtype=torch.bfloat16)
    dq, dk, dv = rc.retention_bwd(q, q, q, [0.9, 0.9], q)
    assert dq.shape == (1, 2, 0, 64) and dk.shape == dq.shape and dv.shape == dq.shape
    e = torch.zeros((0, 2, 16, 64), device="cuda")
    dq, dk, dv = rc.retention_bwd(e, e, e, [0.9, 0.9], e)
    assert dq.shape == e.shape


@pytest.mark.parametrize("gval", [1.0, 0.5, 0.02])
def test_bwd_gamma_extremes(gval, plan):
    w, inp = _inputs(53, "bf16", 1, 2, 900, 64, 64)
    inp["gamma"] = np.full(2, gval, dtype=np.float32)
    _segments(plan, 4)
    got = _run(inp, 64)
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"])
    _check(f"bwd gamma={gval}", got, ref, TOL["bf16"])


def test_bwd_long_sequence_two_heads(plan):
    """The [1, 32, 65536, 128] bf16 shape; the oracle checks heads 0 and 31 in full."""
    _segments(plan, None)
    w = wl.WORKLOADS["ret_fwd_long_bf16"]
    inp = wl.make_inputs(w, 0)
    g = torch.Generator().manual_seed(54)
    do = torch.randn((w.B, w.H, w.T, w.dv), generator=g).to(torch.bfloat16)
    q, k, v, dod = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), do.cuda()
    print("[bwd] long [1,32,65536,128] bf16", flush=True)
    dq, dk, dv = rc.retention_bwd(q, k, v, inp["gamma"], dod, chunk=w.chunk)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        sl = (slice(None), slice(h, h + 1))
        ref = oracle.retention_bwd(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["gamma"][h:h + 1], do[sl],
                                   nthreads=2)
        got = [t[sl].float().cpu().numpy() for t in (dq, dk, dv)]
        _check(f"bwd long head {h}", got, ref, TOL["bf16"])


def test_autograd_wrapper_matches_oracle(plan):
    _segments(plan, None)
    w, inp = _inputs(55, "f32", 2, 2, 300, 64, 128)
    q, k, v = (inp[n].cuda().requires_grad_(True) for n in ("q", "k", "v"))
    out = rc.retention(q, k, v, inp["gamma"], chunk=64)
    (out * inp["do"].cuda()).sum().backward()
    torch.cuda.synchronize()
    ref_out, _ = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"])
    e = oracle.rel_frobenius(out.detach().cpu().numpy(), ref_out)
    print(f"[parity] autograd forward: {e:.3e}", flush=True)
    assert e <= TOL["f32"]
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"])
    _check("autograd", [t.grad.cpu().numpy() for t in (q, k, v)], ref, TOL["f32"])


def test_bwd_deterministic(plan):
    _segments(plan, None)
    w, inp = _inputs(56, "bf16", 1, 4, 2000, 128, 128, 128)
    a = _run(inp, 128)
    b = _run(inp, 128)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "run-to-run gradients differ"


# ------------------------------------------------- backward from the forward's states
def _fwd_workspace(q, v, chunk, inp):
    """Run retention_fwd with an explicit workspace and return that buffer."""
    B, H, T, d_k = q.shape
    n = rc.retention_fwd_workspace_bytes(B, H, T, d_k, v.shape[3], chunk, q.dtype)
    fws = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    return fws, n


def _run_from_fwd(inp, chunk, zero_states=False):
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    fws, n = _fwd_workspace(q, v, chunk, inp)
    rc.retention_fwd(q, k, v, inp["gamma"], chunk=chunk, want_state=False, workspace=fws)
    if zero_states:
        fws.zero_()
    dq, dk, dv = rc.retention_bwd(q, k, v, inp["gamma"], do, chunk=chunk, fwd_workspace=fws)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)], n


@pytest.mark.parametrize("dtype,G", [("bf16", None), ("bf16", 3), ("bf16", 5), ("f32", None), ("f32", 3)])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 1000), (64, 128, 129), (128, 64, 700)])
def test_bwd_from_fwd_small_full(dtype, G, chunk, dk, dv, T, plan):
    w, inp = _inputs(57, dtype, 2, 3, T, dk, dv, chunk)
    _segments(plan, G)
    tag = f"bwd_from_fwd {dtype} G={G} C={chunk} dk={dk} dv={dv} T={T}"
    print(f"[bwd] {tag}", flush=True)
    got, _ = _run_from_fwd(inp, chunk)
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"], nthreads=8)
    _check(tag, got, ref, TOL[dtype])
    # dk and dv take the same walks as retention_bwd; dq differs only in rounding
    plain = _run(inp, chunk)
    assert np.array_equal(got[1], plain[1]) and np.array_equal(got[2], plain[2]), tag
    e = oracle.rel_frobenius(got[0], plain[0].astype(np.float64))
    print(f"[parity] {tag} dq vs retention_bwd: {e:.3e}", flush=True)
    assert e <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_from_fwd_reads_the_given_states(dtype, plan):
    """With the forward's states zeroed, dq loses every earlier segment's share
    and dk, dv are unchanged: the dq walk reads the buffer it is given (segment
    path for bf16, value-slice path for fp32)."""
    _segments(plan, 4)
    w, inp = _inputs(58, dtype, 1, 2, 1024, 64, 64, 64)
    good, n = _run_from_fwd(inp, 64)
    assert n > 0
    bad, _ = _run_from_fwd(inp, 64, zero_states=True)
    assert np.array_equal(good[1], bad[1]) and np.array_equal(good[2], bad[2])
    T1 = 1024 // 4  # the first segment has no earlier states
    assert np.array_equal(good[0][:, :, :T1], bad[0][:, :, :T1])
    assert oracle.rel_frobenius(bad[0], good[0].astype(np.float64)) > 0.05


def test_bwd_from_fwd_without_forward_workspace(plan):
    """A one-segment forward leaves no states: the call equals retention_bwd."""
    _segments(plan, 1)
    w, inp = _inputs(59, "bf16", 2, 2, 500, 128, 64, 128)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    assert rc.retention_fwd_workspace_bytes(2, 2, 500, 128, 64, 128, q.dtype) == 0
    lib = rc.load_library()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g = rc._gamma_array(inp["gamma"], 2)
    ws, nws = rc._workspace(lib.retention_bwd_workspace_bytes(2, 2, 500, 128, 64, 128, rc.RET_BF16), q.device)
    code = lib.retention_bwd_from_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g, 128, do.data_ptr(), None, 0,
                                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), 2, 2, 500, 128, 64, rc.RET_BF16,
                                      rc._ptr(ws), nws, rc._stream(q))
    assert code == 0
    torch.cuda.synchronize()
    plain = _run(inp, 128)
    for x, y in zip((dq, dk, dv), plain):
        assert np.array_equal(x.float().cpu().numpy(), y)


def test_bwd_from_fwd_long_sequence_two_heads(plan):
    """The [1, 32, 65536, 128] bf16 shape as bench.py runs it; heads 0 and 31 in full."""
    _segments(plan, None)
    w = wl.WORKLOADS["ret_fwd_long_bf16"]
    inp = wl.make_inputs(w, 0)
    g = torch.Generator().manual_seed(54)
    do = torch.randn((w.B, w.H, w.T, w.dv), generator=g).to(torch.bfloat16)
    q, k, v, dod = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), do.cuda()
    print("[bwd] from_fwd long [1,32,65536,128] bf16", flush=True)
    fws, n = _fwd_workspace(q, v, w.chunk, inp)
    assert n > 0
    rc.retention_fwd(q, k, v, inp["gamma"], chunk=w.chunk, want_state=False, workspace=fws)
    dq, dk, dv = rc.retention_bwd(q, k, v, inp["gamma"], dod, chunk=w.chunk, fwd_workspace=fws)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        sl = (slice(None), slice(h, h + 1))
        ref = oracle.retention_bwd(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["gamma"][h:h + 1], do[sl],
                                   nthreads=2)
        got = [t[sl].float().cpu().numpy() for t in (dq, dk, dv)]
        _check(f"bwd_from_fwd long head {h}", got, ref, TOL["bf16"])


def test_autograd_wrapper_bf16_shares_states(plan):
    """bf16 through torch.autograd: the forward keeps its workspace for backward."""
    _segments(plan, 3)
    w, inp = _inputs(60, "bf16", 1, 2, 900, 64, 64, 64)
    q, k, v = (inp[n].cuda().requires_grad_(True) for n in ("q", "k", "v"))
    out = rc.retention(q, k, v, inp["gamma"], chunk=64)
    (out.float() * inp["do"].cuda().float()).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["do"])
    _check("autograd bf16", [t.grad.float().cpu().numpy() for t in (q, k, v)], ref, TOL["bf16"])
