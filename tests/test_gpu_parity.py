"""HIP path against the fp64 oracle, element by element (needs a gfx950 GPU).

Tolerances (relative Frobenius error ||x - ref|| / ||ref|| over the compared
tensor): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.
The oracle always sees exactly the values the GPU sees: bf16 inputs are
widened from their rounded values and gamma from its float32 value.
Small cases are compared in full (several chunks and a ragged tail); the
full-size workloads are compared on sampled rows that the oracle evaluates one
at a time from the parallel definition, plus full final states of sampled
heads.
"""
import numpy as np
import pytest
import torch

import oracle
import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl

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


def _report(name, err, tol):
    print(f"[parity] {name}: rel_fro={err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: relative Frobenius error {err:.3e} > {tol:.0e}"


# ------------------------------------------------------------- retention fwd
def test_ret_fwd_tiny_f32_full():
    w, inp = _inputs("ret_fwd_tiny_f32")
    out, fs = _run_fwd(inp, w.chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"])
    _report("tiny f32 out", oracle.rel_frobenius(out, ref), TOL["f32"])
    _report("tiny f32 final_state", oracle.rel_frobenius(fs, ref_s), TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 300), (64, 128, 129), (128, 64, 512)])
def test_ret_fwd_small_full(dtype, chunk, dk, dv, T):
    w, inp = _inputs("ret_fwd_mh_f32", seed=1, B=2, H=3, T=T, dk=dk, dv=dv, chunk=chunk,
                     dtype=dtype, scale=1.0 / np.sqrt(dk))
    out, fs = _run_fwd(inp, chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    tag = f"{dtype} C={chunk} dk={dk} dv={dv} T={T}"
    _report(f"{tag} out", oracle.rel_frobenius(out, ref), TOL[dtype])
    _report(f"{tag} final_state", oracle.rel_frobenius(fs, ref_s), TOL[dtype])


def test_ret_fwd_mh_f32_full_size():
    w, inp = _inputs("ret_fwd_mh_f32")
    out, fs = _run_fwd(inp, w.chunk)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=16)
    _report("mh f32 [4,8,2048,64] out", oracle.rel_frobenius(out, ref), TOL["f32"])
    _report("mh f32 final_state", oracle.rel_frobenius(fs, ref_s), TOL["f32"])
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


def test_ret_fwd_long_bf16_full_size_sampled():
    w, inp = _inputs("ret_fwd_long_bf16")
    out, fs = _run_fwd(inp, w.chunk)
    rng = np.random.default_rng(0)
    rows = _sample_rows(rng, w.B, w.H, w.T, 48)
    ref_rows = _rows_by_head(oracle.retention_rows, inp, rows, with_gamma=True)
    got = np.stack([out[b, h, t] for b, h, t in rows])
    _report("long bf16 [1,32,65536,128] sampled rows", oracle.rel_frobenius(got, ref_rows), TOL["bf16"])
    for h in (0, 31):
        _, ref_s = oracle.retention_recurrent(inp["q"][:, h:h + 1], inp["k"][:, h:h + 1],
                                              inp["v"][:, h:h + 1], inp["gamma"][h:h + 1])
        _report(f"long bf16 final_state head {h}", oracle.rel_frobenius(fs[:, h:h + 1], ref_s),
                TOL["bf16"])


def test_ret_fwd_chunk_invariance_and_determinism():
    w, inp = _inputs("ret_fwd_mh_f32", seed=2, B=1, H=4, T=700)
    o64, s64 = _run_fwd(inp, 64)
    o128, s128 = _run_fwd(inp, 128)
    _report("chunk 64 vs 128 out", oracle.rel_frobenius(o64, o128), TOL["f32"])
    _report("chunk 64 vs 128 state", oracle.rel_frobenius(s64, s128), TOL["f32"])
    o64b, s64b = _run_fwd(inp, 64)
    assert np.array_equal(o64, o64b) and np.array_equal(s64, s64b), "run-to-run results differ"


def test_ret_fwd_gamma_one_is_masked_linear_attention():
    w, inp = _inputs("ret_fwd_mh_f32", seed=3, B=1, H=2, T=300, gamma="one")
    out, fs = _run_fwd(inp, 64)
    q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    _report("gamma=1 masked QK^T V", oracle.rel_frobenius(out, ref), TOL["f32"])
    _report("gamma=1 final state = K^T V", oracle.rel_frobenius(fs, np.swapaxes(k, -1, -2) @ v),
            TOL["f32"])


@pytest.mark.parametrize("T", [0, 1, 5, 64, 65])
def test_ret_fwd_edge_lengths(T):
    w, inp = _inputs("ret_fwd_mh_f32", seed=4, B=1, H=2, T=T)
    out, fs = _run_fwd(inp, 64)
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"])
    if T == 0:
        assert out.size == 0 and np.all(fs == 0.0)
        return
    _report(f"T={T} out", oracle.rel_frobenius(out, ref), TOL["f32"])
    _report(f"T={T} state", oracle.rel_frobenius(fs, ref_s), TOL["f32"])


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
    _report(f"decode {dtype} {dk}x{dv} out", oracle.rel_frobenius(outs[-1], ref_o), TOL[dtype])
    _report(f"decode {dtype} {dk}x{dv} state", oracle.rel_frobenius(state.cpu().numpy(), ref_s), 1e-4)


def test_decode_full_size_1000_steps_sampled():
    w, inp = _inputs("decode_bf16")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    state = _dev(inp["state"]).clone()
    for _ in range(w.steps):
        out = rc.retention_decode_step(q, k, v, inp["gamma"], state)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    pairs = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(12)} |
                   {(0, 0), (w.B - 1, w.H - 1)})
    st = state.cpu().numpy()
    o = out.float().cpu().numpy()
    for n, h in pairs:
        ro, rs = oracle.decode_steps(inp["q"][n:n + 1, h:h + 1], inp["k"][n:n + 1, h:h + 1],
                                     inp["v"][n:n + 1, h:h + 1], inp["gamma"][h:h + 1],
                                     inp["state"][n:n + 1, h:h + 1], nsteps=w.steps)
        e_s = oracle.rel_frobenius(st[n:n + 1, h:h + 1], rs)
        e_o = oracle.rel_frobenius(o[n:n + 1, h:h + 1], ro)
        print(f"[parity] decode 1000 steps seq {n} head {h}: state {e_s:.2e} out {e_o:.2e}", flush=True)
        assert e_s <= 1e-4 and e_o <= TOL["bf16"]


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
        _report(f"handoff step {s}", oracle.rel_frobenius(o.cpu().numpy(), full[:, :, T0 + s].cpu().numpy()),
                TOL["f32"])


# ------------------------------------------------------------- linear attention
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 300), (128, 64, 257), (64, 128, 128)])
def test_linattn_small_full(dtype, dk, dv, T):
    w, inp = _inputs("linattn_elu1_bf16", seed=7, B=2, H=3, T=T, dk=dk, dv=dv, dtype=dtype)
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    out = rc.linear_attn_fwd(q, k, v).float().cpu().numpy()
    ref, _, _ = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    _report(f"linattn {dtype} dk={dk} dv={dv} T={T}", oracle.rel_frobenius(out, ref), TOL[dtype])


def test_linattn_full_size_sampled():
    w, inp = _inputs("linattn_elu1_bf16")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    out = rc.linear_attn_fwd(q, k, v).float().cpu().numpy()
    rng = np.random.default_rng(2)
    rows = _sample_rows(rng, w.B, w.H, w.T, 64)
    ref_rows = _rows_by_head(oracle.linattn_rows, inp, rows, with_gamma=False)
    got = np.stack([out[b, h, t] for b, h, t in rows])
    _report("linattn [8,16,8192,64] sampled rows", oracle.rel_frobenius(got, ref_rows), TOL["bf16"])


def test_linattn_constant_values_give_constant_outputs():
    w, inp = _inputs("linattn_elu1_bf16", seed=8, B=1, H=2, T=300, dtype="f32")
    u = torch.randn(w.dv)
    v = u.expand(1, 2, 300, w.dv).contiguous()
    out = rc.linear_attn_fwd(_dev(inp["q"]), _dev(inp["k"]), _dev(v), eps=0.0).cpu().numpy()
    _report("constant values", oracle.rel_frobenius(out, v.numpy()), TOL["f32"])


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
    _report(f"256 heads {dtype} out", oracle.rel_frobenius(out, ref), TOL[dtype])
    _report(f"256 heads {dtype} final_state", oracle.rel_frobenius(fs, ref_s), TOL[dtype])

    wd, dinp = _inputs("decode_bf16", seed=10, B=1, H=H, dk=64, dv=64, dtype=dtype)
    state = torch.from_numpy(fs).cuda()
    q, k, v = (_dev(dinp[n]) for n in ("q", "k", "v"))
    for _ in range(2):
        o = rc.retention_decode_step(q, k, v, inp["gamma"], state)
    torch.cuda.synchronize()
    ref_o, ref_st = oracle.decode_steps(dinp["q"], dinp["k"], dinp["v"], inp["gamma"], fs, nsteps=2)
    _report(f"256 heads {dtype} decode out", oracle.rel_frobenius(o.float().cpu().numpy(), ref_o), TOL[dtype])
    _report(f"256 heads {dtype} decode state", oracle.rel_frobenius(state.cpu().numpy(), ref_st), 1e-4)

    g = torch.Generator().manual_seed(11)
    do = torch.randn((1, H, 200, 64), generator=g).to(wl.torch_dtype(dtype))
    dq, dk, dv = rc.retention_bwd(*(_dev(inp[n]) for n in ("q", "k", "v")), inp["gamma"], do.cuda(), chunk=64)
    torch.cuda.synchronize()
    ref_g = oracle.retention_bwd(inp["q"], inp["k"], inp["v"], inp["gamma"], do, nthreads=8)
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref_g):
        _report(f"256 heads {dtype} {name}", oracle.rel_frobenius(x.float().cpu().numpy(), r), TOL[dtype])
