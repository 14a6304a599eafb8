"""Forwards from an initial state and the elu+1 decode step against the fp64
oracle (needs a gfx950 GPU).

retention_fwd_from_state and linear_attn_fwd_from_state continue a sequence
from the state (and normaliser) after earlier tokens; linear_attn_decode_step
is the one-token step of causal linear attention.  Every case compares the
outputs and the returned state with the oracle run from the same initial
state, on both forward paths (value slices; segments with several segment
counts), fp32 and bf16, every (dk, dv) pair, ragged lengths, and chunked
prefills whose pieces are chained through the returned state.
Tolerances: relative Frobenius error 1e-4 for fp32, 2e-2 for bf16 inputs
(fp32 accumulation); decode states, fp32 throughout, 1e-4.
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


def _path(plan, path, segments):
    plan(path=path, segments=segments)


_report = parity.check


def _ret_inputs(seed, dtype, B, H, T, dk, dv, chunk):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(B=B, H=H, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype,
                                              scale=1.0 / np.sqrt(dk))
    inp = wl.make_inputs(w, seed)
    rng = np.random.default_rng(seed + 1000)
    inp["S0"] = torch.from_numpy((rng.standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32))
    return w, inp


# ------------------------------------------------------------- retention from a state
PATHS = [("f32", "slice", None), ("bf16", "slice", None), ("bf16", "segment", 1), ("bf16", "segment", 3),
         ("bf16", "segment", 7)]


@pytest.mark.parametrize("dtype,path,G", PATHS)
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 1000), (64, 128, 129), (128, 64, 700)])
def test_ret_fwd_from_state_full(dtype, path, G, chunk, dk, dv, T, plan):
    w, inp = _ret_inputs(31, dtype, 2, 3, T, dk, dv, chunk)
    _path(plan, path, G)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    print(f"[state] retention {dtype} {path} G={G} C={chunk} dk={dk} dv={dv} T={T}", flush=True)
    out, fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=chunk, initial_state=inp["S0"].cuda())
    torch.cuda.synchronize()
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], init_state=inp["S0"],
                                            nthreads=8)
    tag = f"from-state {dtype} {path} G={G} C={chunk} dk={dk} dv={dv} T={T}"
    _report(tag + " out", out.float().cpu().numpy(), ref, TOL[dtype])
    _report(tag + " final", fs.cpu().numpy(), ref_s, TOL[dtype])


@pytest.mark.parametrize("dtype,path,G", PATHS)
def test_ret_fwd_from_state_zero_length_copies_state(dtype, path, G, plan):
    w, inp = _ret_inputs(32, dtype, 1, 2, 0, 128, 64, 64)
    _path(plan, path, G)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    _, fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=64, initial_state=inp["S0"].cuda())
    torch.cuda.synchronize()
    assert torch.equal(fs.cpu(), inp["S0"])


@pytest.mark.parametrize("gval", [1.0, 0.5])
def test_ret_fwd_from_state_gamma_extremes(gval, plan):
    w, inp = _ret_inputs(33, "bf16", 1, 2, 1500, 64, 64, 64)
    inp["gamma"] = np.full(2, gval, dtype=np.float32)
    _path(plan, "segment", 6)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out, fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=64, initial_state=inp["S0"].cuda())
    torch.cuda.synchronize()
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], init_state=inp["S0"])
    _report(f"from-state gamma={gval} out", out.float().cpu().numpy(), ref, TOL["bf16"])
    _report(f"from-state gamma={gval} final", fs.cpu().numpy(), ref_s, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ret_chunked_prefill_matches_one_call(dtype, plan):
    """A sequence run in pieces, each from the previous piece's final state."""
    w, inp = _ret_inputs(34, dtype, 1, 4, 3000, 128, 128, 128)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    cuts = [0, 1000, 1777, 1800, 3000]
    outs, state = [], None  # the first piece starts from zero (the plain entry point)
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, state = rc.retention_fwd(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                                    v[:, :, a:b].contiguous(), inp["gamma"], chunk=128, initial_state=state)
        outs.append(o)
    whole, ws = rc.retention_fwd(q, k, v, inp["gamma"], chunk=128)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy()
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    _report(f"chunked prefill {dtype} out", got, ref, TOL[dtype])
    _report(f"chunked prefill {dtype} final", state.cpu().numpy(), ref_s, TOL[dtype])
    _report(f"chunked prefill {dtype} vs one call", got, whole.float().cpu().numpy(), TOL[dtype])


# ------------------------------------------------------------- linear attention from a state
def _lin_inputs(seed, dtype, B, H, T, dk, dv, prefix=150):
    """Inputs and an initial (S0, z0) that is the oracle's state after a
    random prefix of `prefix` tokens, rounded to float32 (what the GPU reads)."""
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=B, H=H, T=T + prefix, dk=dk, dv=dv, dtype=dtype)
    full = wl.make_inputs(w, seed)
    inp = {n: full[n][:, :, prefix:].contiguous() for n in ("q", "k", "v")}
    _, S0, z0 = oracle.linattn_recurrent(full["q"][:, :, :prefix], full["k"][:, :, :prefix],
                                         full["v"][:, :, :prefix])
    inp["S0"] = torch.from_numpy(S0.astype(np.float32))
    inp["z0"] = torch.from_numpy(z0.astype(np.float32))
    return inp


LIN_PATHS = [("f32", "slice", None), ("bf16", "slice", None), ("bf16", "segment", 1), ("bf16", "segment", 4)]


@pytest.mark.parametrize("dtype,path,G", LIN_PATHS)
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 300), (128, 64, 1000), (64, 128, 129), (128, 128, 700)])
def test_linattn_from_state_full(dtype, path, G, dk, dv, T, plan):
    inp = _lin_inputs(41, dtype, 2, 2, T, dk, dv)
    _path(plan, path, G)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    print(f"[state] linattn {dtype} {path} G={G} dk={dk} dv={dv} T={T}", flush=True)
    out, S, z = rc.linear_attn_fwd(q, k, v, initial_state=(inp["S0"].cuda(), inp["z0"].cuda()),
                                   return_state=True)
    torch.cuda.synchronize()
    ref, rS, rz = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], init_S=inp["S0"], init_z=inp["z0"],
                                           nthreads=8)
    tag = f"linattn from-state {dtype} {path} G={G} dk={dk} dv={dv} T={T}"
    _report(tag + " out", out.float().cpu().numpy(), ref, TOL[dtype])
    _report(tag + " S", S.cpu().numpy(), rS, TOL[dtype])
    _report(tag + " z", z.cpu().numpy(), rz, TOL[dtype])


@pytest.mark.parametrize("dtype,path,G", LIN_PATHS)
def test_linattn_returns_state_from_zero(dtype, path, G, plan):
    inp = _lin_inputs(42, dtype, 1, 3, 500, 64, 64)
    _path(plan, path, G)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out, S, z = rc.linear_attn_fwd(q, k, v, return_state=True)
    plain = rc.linear_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    ref, rS, rz = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"])
    _report(f"linattn zero-start {dtype} {path} out", out.float().cpu().numpy(), ref, TOL[dtype])
    _report(f"linattn zero-start {dtype} {path} S", S.cpu().numpy(), rS, TOL[dtype])
    _report(f"linattn zero-start {dtype} {path} z", z.cpu().numpy(), rz, TOL[dtype])
    assert torch.equal(out, plain), "returning the state changed the output"


def test_linattn_from_state_zero_length_copies_state(plan):
    inp = _lin_inputs(43, "bf16", 1, 2, 0, 128, 64)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    _, S, z = rc.linear_attn_fwd(q, k, v, initial_state=(inp["S0"].cuda(), inp["z0"].cuda()), return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), inp["S0"]) and torch.equal(z.cpu(), inp["z0"])


# ------------------------------------------------------------- elu+1 decode step
@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 128, 64), ("bf16", 64, 128),
                                         ("bf16", 128, 128)])
def test_linattn_decode_small(dtype, dk, dv):
    inp = _lin_inputs(44, dtype, 5, 3, 1, dk, dv, prefix=60)
    q, k, v = (inp[n][:, :, 0].contiguous() for n in ("q", "k", "v"))
    S, z = inp["S0"].cuda().clone(), inp["z0"].cuda().clone()
    for _ in range(3):
        out = rc.linear_attn_decode_step(q.cuda(), k.cuda(), v.cuda(), S, z)
    torch.cuda.synchronize()
    ro, rS, rz = oracle.linattn_decode_steps(q, k, v, inp["S0"], inp["z0"], nsteps=3)
    _report(f"phi decode {dtype} {dk}x{dv} out", out.float().cpu().numpy(), ro, TOL[dtype])
    _report(f"phi decode {dtype} {dk}x{dv} S", S.cpu().numpy(), rS, 1e-4)
    _report(f"phi decode {dtype} {dk}x{dv} z", z.cpu().numpy(), rz, 1e-4)


def test_linattn_decode_full_size_1000_steps_whole_tensor():
    """256 sequences x 32 heads, 128 x 128 state, 1000 steps of one token:
    every S, z and output after the last step against the oracle's 1000
    steps, 8 heads (2048 pairs) at a time."""
    N, H, d, steps = 256, 32, 128, 1000
    g = torch.Generator().manual_seed(45)
    q, k, v = (torch.randn((N, H, d), generator=g) / np.sqrt(d)).to(torch.bfloat16), \
        (torch.randn((N, H, d), generator=g) / np.sqrt(d)).to(torch.bfloat16), \
        (torch.randn((N, H, d), generator=g) / np.sqrt(d)).to(torch.bfloat16)
    # a state as after about 100 tokens: z ~ 100 phi(k), S ~ sum of 100 phi(k) v^T
    z0 = (100.0 + 10.0 * torch.rand((N, H, d), generator=g)).float()
    S0 = (torch.randn((N, H, d, d), generator=g) * 10.0).float()
    S, z = S0.cuda(), z0.cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for _ in range(steps):
        out = rc.linear_attn_decode_step(qd, kd, vd, S, z)
    torch.cuda.synchronize()
    st, zt, o = S.cpu().numpy(), z.cpu().numpy(), out.float().cpu().numpy()
    acc_s = parity.HeadGroups("phi decode 1000 steps S", 1e-4)
    acc_z = parity.HeadGroups("phi decode 1000 steps z", 1e-4)
    acc_o = parity.HeadGroups("phi decode 1000 steps out", TOL["bf16"])
    for h0 in range(0, H, 8):
        sl = (slice(None), slice(h0, h0 + 8))
        ro, rS, rz = oracle.linattn_decode_steps(q[sl], k[sl], v[sl], S0[sl], z0[sl], nsteps=steps, nthreads=16)
        per = acc_s.add(st[sl], rS, h0)
        acc_z.add(zt[sl], rz, h0)
        acc_o.add(o[sl], ro, h0)
        print(f"[parity] phi decode heads {h0}..{h0 + 7}: worst S per head " +
              " ".join(f"{e:.1e}" for e in per.max(axis=0)), flush=True)
    acc_s.finish()
    acc_z.finish()
    acc_o.finish()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linattn_prefill_then_decode_handoff(dtype, plan):
    """Prefill T0 tokens, then decode the rest one token at a time: the
    decoded outputs are the last rows of one forward over all tokens."""
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=2, H=2, T=1300, dk=64, dv=64, dtype=dtype)
    inp = wl.make_inputs(w, 46)
    T0, n = 1290, 10
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    _, S, z = rc.linear_attn_fwd(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                                 return_state=True)
    outs = []
    for s in range(n):
        outs.append(rc.linear_attn_decode_step(q[:, :, T0 + s].contiguous(), k[:, :, T0 + s].contiguous(),
                                               v[:, :, T0 + s].contiguous(), S, z))
    torch.cuda.synchronize()
    ref, rS, rz = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    got = torch.stack(outs, dim=2).float().cpu().numpy()
    _report(f"phi handoff {dtype} decoded rows", got, ref[:, :, T0:], TOL[dtype])
    _report(f"phi handoff {dtype} S", S.cpu().numpy(), rS, TOL[dtype])
    _report(f"phi handoff {dtype} z", z.cpu().numpy(), rz, TOL[dtype])


def test_linattn_chunked_prefill_matches_one_call(plan):
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=2, H=4, T=3000)
    inp = wl.make_inputs(w, 47)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    cuts = [0, 640, 700, 2222, 3000]
    outs, st = [], None
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, S, z = rc.linear_attn_fwd(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                                     v[:, :, a:b].contiguous(), initial_state=st, return_state=True)
        st = (S, z)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy()
    ref, rS, rz = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    _report("linattn chunked prefill out", got, ref, TOL["bf16"])
    _report("linattn chunked prefill S", st[0].cpu().numpy(), rS, TOL["bf16"])
    _report("linattn chunked prefill z", st[1].cpu().numpy(), rz, TOL["bf16"])
