"""HIP path against the fp64 oracle, element by element (needs a gfx950 GPU).

Tolerances (relative Frobenius error ||x - ref|| / ||ref|| over the compared
tensor, and over each (b, h) slice of it): 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 accumulation.  The oracle always sees exactly the values the
GPU sees: bf16 inputs are widened from their rounded values and gamma from its
float32 value.  Every case is compared in full, the full-size workloads too:
the oracle's recurrent form runs over every head of the [1,32,65536,128]
forward, the [8,16,8192,64] linear attention and the 1000-step decode of 256 x
32 states, one head group at a time.  Sampled rows from the parallel definition
(an independent formula) back up the two long forwards.
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


def _dev(x):
    return x.cuda() if isinstance(x, torch.Tensor) else x


def _inputs(name, seed=0, **over):
    w = wl.WORKLOADS[name].with_(**over) if over else wl.WORKLOADS[name]
    return w, wl.make_inputs(w, seed)


def _run_fwd(inp, chunk):
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    out, fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fs.cpu().numpy()


_check = parity.check


# ------------------------------------------------------------- retention fwd
def test_ret_fwd_tiny_f32_full():
    w, inp = _inputs("ret_fwd_tiny_f32")
    out, fs = _run_fwd(inp, w.chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"])
    _check("tiny f32 out", out, ref, TOL["f32"])
    _check("tiny f32 final_state", fs, ref_s, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 300), (64, 128, 129), (128, 64, 512)])
def test_ret_fwd_small_full(dtype, chunk, dk, dv, T):
    w, inp = _inputs("ret_fwd_mh_f32", seed=1, B=2, H=3, T=T, dk=dk, dv=dv, chunk=chunk,
                     dtype=dtype, scale=1.0 / np.sqrt(dk))
    out, fs = _run_fwd(inp, chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    tag = f"{dtype} C={chunk} dk={dk} dv={dv} T={T}"
    _check(f"{tag} out", out, ref, TOL[dtype])
    _check(f"{tag} final_state", fs, ref_s, TOL[dtype])


def test_ret_fwd_mh_f32_full_size():
    w, inp = _inputs("ret_fwd_mh_f32")
    out, fs = _run_fwd(inp, w.chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=16)
    _check("mh f32 [4,8,2048,64] out", out, ref, TOL["f32"])
    _check("mh f32 final_state", fs, ref_s, TOL["f32"])
    # per-head diagnostic
    worst = max(oracle.rel_frobenius(out[:, h], ref[:, h]) for h in range(w.H))
    print(f"[parity] mh f32 worst head rel_fro={worst:.3e}", flush=True)


def _sample_rows(rng, B, H, T, n):
    rows = []
    for _ in range(n):
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T))))
    # always include the first, chunk-boundary and last rows
    for t in (0, 1, 127, 128, 129, T - 1):
        if t < T:
            rows.append((B - 1, H - 1, t))
    return rows


def _rows_by_head(fn, inp, rows, with_gamma):
    """Evaluate oracle rows one (b, h) slice at a time (keeps fp64 copies small)."""
    out = np.zeros((len(rows), inp["v"].shape[-1]))
    groups = {}
    for i, (b, h, t) in enumerate(rows):
        groups.setdefault((b, h), []).append((i, t))
    for (b, h), items in groups.items():
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = [inp["q"][sl], inp["k"][sl], inp["v"][sl]]
        if with_gamma:
            args.append(inp["gamma"][h:h + 1])
        res = fn(*args, [(0, 0, t) for _, t in items], nthreads=16)
        for (i, _), r in zip(items, res):
            out[i] = r
    return out


def test_ret_fwd_long_bf16_full_size_whole_tensor():
    """[1, 32, 65536, 128] bf16, chunk 128, in the launch configuration the
    benchmark times: every output row and all 32 final states against the
    recurrent oracle, 8 heads at a time."""
    w, inp = _inputs("ret_fwd_long_bf16")
    out, fs = _run_fwd(inp, w.chunk)
    acc_o = parity.HeadGroups("long bf16 [1,32,65536,128] out", TOL["bf16"])
    acc_s = parity.HeadGroups("long bf16 [1,32,65536,128] final_state", TOL["bf16"])
    for h0 in range(0, w.H, 8):
        sl = slice(h0, h0 + 8)
        ref, ref_s = oracle.retention_recurrent(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl],
                                                inp["gamma"][sl], nthreads=16)
        per = acc_o.add(out[:, sl], ref, h0)
        acc_s.add(fs[:, sl], ref_s, h0)
        print(f"[parity] long bf16 heads {h0}..{h0 + 7}: per-head out " + " ".join(f"{e:.2e}" for e in per[0]),
              flush=True)
    acc_o.finish()
    acc_s.finish()
    # rows from the parallel definition, an independent formula, at chunk and segment edges
    rng = np.random.default_rng(0)
    rows = _sample_rows(rng, w.B, w.H, w.T, 48)
    ref_rows = _rows_by_head(oracle.retention_rows, inp, rows, with_gamma=True)
    got = np.stack([out[b, h, t] for b, h, t in rows])
    _check("long bf16 sampled rows (parallel form)", got, ref_rows, TOL["bf16"])


def test_ret_fwd_chunk_invariance_and_determinism():
    w, inp = _inputs("ret_fwd_mh_f32", seed=2, B=1, H=4, T=700)
    o64, s64 = _run_fwd(inp, 64)
    o128, s128 = _run_fwd(inp, 128)
    _check("chunk 64 vs 128 out", o64, o128, TOL["f32"])
    _check("chunk 64 vs 128 state", s64, s128, TOL["f32"])
    o64b, s64b = _run_fwd(inp, 64)
    assert np.array_equal(o64, o64b) and np.array_equal(s64, s64b), "run-to-run results differ"


def test_ret_fwd_gamma_one_is_masked_linear_attention():
    w, inp = _inputs("ret_fwd_mh_f32", seed=3, B=1, H=2, T=300, gamma="one")
    out, fs = _run_fwd(inp, 64)
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    _check("gamma=1 masked QK^T V", out, ref, TOL["f32"])
    _check("gamma=1 final state = K^T V", fs, np.swapaxes(k, -1, -2) @ v, TOL["f32"])


@pytest.mark.parametrize("T", [0, 1, 5, 64, 65])
def test_ret_fwd_edge_lengths(T):
    w, inp = _inputs("ret_fwd_mh_f32", seed=4, B=1, H=2, T=T)
    out, fs = _run_fwd(inp, 64)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"])
    if T == 0:
        assert out.size == 0 and np.all(fs == 0.0)
        return
    _check(f"T={T} out", out, ref, TOL["f32"])
    _check(f"T={T} state", fs, ref_s, TOL["f32"])


def test_ret_fwd_empty_batch_is_noop():
    q = torch.zeros((0, 2, 16, 64), device="cuda")
    out, fs = rc.retention_fwd(q, q, q, [0.9, 0.9])
    assert out.shape == (0, 2, 16, 64) and fs.shape == (0, 2, 64, 64)


# ------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 128, 64), ("bf16", 64, 128),
                                         ("bf16", 128, 128)])
def test_decode_small(dtype, dk, dv):
    w, inp = _inputs("decode_bf16", seed=5, B=5, H=3, dk=dk, dv=dv, dtype=dtype)
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    state = _dev(inp["state"]).clone()
    outs = []
    for _ in range(3):
        outs.append(rc.retention_decode_step(q, k, v, inp["gamma"], state).float().cpu().numpy())
    torch.cuda.synchronize()
    ref_o, ref_s = oracle.decode_steps(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["state"], nsteps=3)
    _check(f"decode {dtype} {dk}x{dv} out", outs[-1], ref_o, TOL[dtype])
    _check(f"decode {dtype} {dk}x{dv} state", state.cpu().numpy(), ref_s, 1e-4)


def test_decode_full_size_1000_steps_whole_tensor():
    """256 sequences x 32 heads of 128 x 128 fp32 states, 1000 steps of one
    bf16 token: every state and every output after the last step against the
    oracle's 1000 steps, 8 heads (2048 states) at a time."""
    w, inp = _inputs("decode_bf16")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    state = _dev(inp["state"]).clone()
    for _ in range(w.steps):
        out = rc.retention_decode_step(q, k, v, inp["gamma"], state)
    torch.cuda.synchronize()
    st = state.cpu().numpy()
    o = out.float().cpu().numpy()
    acc_s = parity.HeadGroups("decode 1000 steps [256,32,128,128] state", 1e-4)
    acc_o = parity.HeadGroups("decode 1000 steps [256,32,128] out", TOL["bf16"])
    for h0 in range(0, w.H, 8):
        sl = (slice(None), slice(h0, h0 + 8))
        ro, rs = oracle.decode_steps(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["gamma"][h0:h0 + 8],
                                     inp["state"][sl], nsteps=w.steps, nthreads=16)
        per = acc_s.add(st[sl], rs, h0)
        acc_o.add(o[sl], ro, h0)
        print(f"[parity] decode heads {h0}..{h0 + 7}: worst state per head " +
              " ".join(f"{e:.1e}" for e in per.max(axis=0)), flush=True)
    acc_s.finish()
    acc_o.finish()


def test_prefill_then_decode_handoff():
    w, inp = _inputs("ret_fwd_mh_f32", seed=6, B=2, H=2, T=200)
    T0, n = 190, 10
    q, k, v = (_dev(inp[x]) for x in ("q", "k", "v"))
    full, _ = rc.retention_fwd(q, k, v, inp["gamma"], chunk=64)
    _, state = rc.retention_fwd(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(),
                                v[:, :, :T0].contiguous(), inp["gamma"], chunk=64)
    for s in range(n):
        o = rc.retention_decode_step(q[:, :, T0 + s].contiguous(), k[:, :, T0 + s].contiguous(),
                                     v[:, :, T0 + s].contiguous(), inp["gamma"], state)
        _check(f"handoff step {s}", o.cpu().numpy(), full[:, :, T0 + s].cpu().numpy(), TOL["f32"])


# ------------------------------------------------------------- linear attention
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 300), (128, 64, 257), (64, 128, 128)])
def test_linattn_small_full(dtype, dk, dv, T):
    w, inp = _inputs("linattn_elu1_bf16", seed=7, B=2, H=3, T=T, dk=dk, dv=dv, dtype=dtype)
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    out = rc.linear_attn_fwd(q, k, v).float().cpu().numpy()
    ref, _, _ = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    _check(f"linattn {dtype} dk={dk} dv={dv} T={T}", out, ref, TOL[dtype])


def test_linattn_full_size_whole_tensor():
    """[8, 16, 8192, 64] bf16 elu+1 linear attention: every output row against
    the recurrent oracle, plus rows from the parallel form."""
    w, inp = _inputs("linattn_elu1_bf16")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    out = rc.linear_attn_fwd(q, k, v).float().cpu().numpy()
    acc = parity.HeadGroups("linattn [8,16,8192,64] out", TOL["bf16"])
    for h0 in range(0, w.H, 8):
        sl = (slice(None), slice(h0, h0 + 8))
        ref, _, _ = oracle.linattn_recurrent(inp["q"][sl], inp["k"][sl], inp["v"][sl], nthreads=16)
        per = acc.add(out[sl], ref, h0)
        print(f"[parity] linattn heads {h0}..{h0 + 7}: worst per head " +
              " ".join(f"{e:.2e}" for e in per.max(axis=0)), flush=True)
    acc.finish()
    rng = np.random.default_rng(2)
    rows = _sample_rows(rng, w.B, w.H, w.T, 64)
    ref_rows = _rows_by_head(oracle.linattn_rows, inp, rows, with_gamma=False)
    got = np.stack([out[b, h, t] for b, h, t in rows])
    _check("linattn sampled rows (parallel form)", got, ref_rows, TOL["bf16"])


def test_linattn_constant_values_give_constant_outputs():
    w, inp = _inputs("linattn_elu1_bf16", seed=8, B=1, H=2, T=300, dtype="f32")
    u = torch.randn(w.dv)
    v = u.expand(1, 2, 300, w.dv).contiguous()
    out = rc.linear_attn_fwd(_dev(inp["q"]), _dev(inp["k"]), _dev(v), eps=0.0).cpu().numpy()
    _check("constant values", out, v.numpy(), TOL["f32"])


# ------------------------------------------------------------- the largest head count
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_max_heads_each_with_its_own_gamma(dtype):
    """256 heads, the most one call takes, each with its own decay
    1 - 2^(-5 - 4h/255): the forward (value-slice path for fp32, segment path
    for bf16, ragged tail), decode steps from the forward's final state, and the
    gradients.  A head reading another head's decay would fail here."""
    H = 256
    w, inp = _inputs("ret_fwd_long_bf16", seed=9, B=1, H=H, T=200, dk=64, dv=64, chunk=64, dtype=dtype)
    assert len(set(inp["gamma"].tolist())) == H
    out, fs = _run_fwd(inp, 64)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    _check(f"256 heads {dtype} out", out, ref, TOL[dtype])
    _check(f"256 heads {dtype} final_state", fs, ref_s, TOL[dtype])

    wd, dinp = _inputs("decode_bf16", seed=10, B=1, H=H, dk=64, dv=64, dtype=dtype)
    state = torch.from_numpy(fs).cuda()
    q, k, v = (_dev(dinp[n]) for n in ("q", "k", "v"))
    for _ in range(2):
        o = rc.retention_decode_step(q, k, v, inp["gamma"], state)
    torch.cuda.synchronize()
    ref_o, ref_st = oracle.decode_steps(dinp["q"], dinp["k"], dinp["v"], inp["gamma"], fs, nsteps=2)
    _check(f"256 heads {dtype} decode out", o.float().cpu().numpy(), ref_o, TOL[dtype])
    _check(f"256 heads {dtype} decode state", state.cpu().numpy(), ref_st, 1e-4)

    g = torch.Generator().manual_seed(11)
    do = torch.randn((1, H, 200, 64), generator=g).to(wl.torch_dtype(dtype))
    dq, dk, dv = rc.retention_bwd(*(_dev(inp[n]) for n in ("q", "k", "v")), inp["gamma"], do.cuda(), chunk=64)
    torch.cuda.synchronize()
    ref_g = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], do, nthreads=8)
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref_g):
        _check(f"256 heads {dtype} {name}", x.float().cpu().numpy(), r, TOL[dtype])
