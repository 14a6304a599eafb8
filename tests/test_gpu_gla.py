"""Gated linear attention (gla_fwd, per-token per-key-channel gates) against
the fp64 oracle (needs a gfx950 GPU).

The oracle runs S_t = diag(exp(lg_t)) S_{t-1} + k_t^T v_t token by token; the
kernel walks 64-token chunks with exponentials of running log-gate sums.
Gates are log-sigmoids of Gaussian logits, from slow forgetting (gate about
0.95) to fast (about 0.1), plus isolated near-resets; every (dk, dv) pair,
ragged lengths, one and two value slices, the final state, and the two
special cases the pages name (a constant gate is retention, a unit gate linear
attention); bf16 q, k, v and out (fp32 gates and arithmetic) on the same
cases; gates above 1 are taken as 1.
Tolerance: relative Frobenius error 1e-4 (fp32), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOLS = {"f32": 1e-4, "bf16": 2e-2}


def _inputs(seed, B, H, T, dk, dv, mu, dtype="f32"):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, scale=1.0 / np.sqrt(dk))
    inp = wl.make_inputs(w, seed)
    g = torch.Generator().manual_seed(seed + 900)
    inp["lg"] = torch.nn.functional.logsigmoid(torch.randn((B, H, T, dk), generator=g) + mu).float()
    return w, inp


def _run(inp):
    q, k, v, lg = (inp[n].cuda() for n in ("q", "k", "v", "lg"))
    out, fs = rc.gla_fwd(q, k, v, lg)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fs.cpu().numpy()


def _check(tag, out, fs, inp, tol=TOL):
    ref, ref_s = oracle.gla_recurrent(inp["q"], inp["k"], inp["v"], inp["lg"], nthreads=8)
    parity.check(f"{tag} out", out, ref, tol)
    parity.check(f"{tag} state", fs, ref_s, tol)


@pytest.mark.parametrize("mu", [3.0, 0.0, -2.0])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 300), (64, 128, 129), (128, 64, 200)])
def test_gla_small_full(mu, dk, dv, T):
    w, inp = _inputs(71, 2, 3, T, dk, dv, mu)
    out, fs = _run(inp)
    _check(f"gla mu={mu} dk={dk} dv={dv} T={T}", out, fs, inp)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 129])
def test_gla_short_and_ragged(T):
    w, inp = _inputs(72, 1, 2, T, 64, 64, 1.0)
    out, fs = _run(inp)
    _check(f"gla short T={T}", out, fs, inp)


def test_gla_near_reset():
    """Isolated gates of e^-20 on all channels: the state is nearly erased there."""
    w, inp = _inputs(73, 1, 2, 400, 64, 64, 2.0)
    inp["lg"][:, :, 100] = -20.0
    inp["lg"][:, 1, 257] = -20.0
    out, fs = _run(inp)
    _check("gla near reset", out, fs, inp)


def test_gla_wide_slices():
    """Enough (b, h) pairs for 64-column slices (the other slice width)."""
    w, inp = _inputs(74, 4, 64, 140, 64, 64, 1.0)
    out, fs = _run(inp)
    _check("gla 256 heads", out, fs, inp)


def test_gla_special_cases_match_retention():
    w, inp = _inputs(75, 2, 3, 500, 64, 64, 0.0)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    gam = np.array([0.9, 0.99, 1.0], dtype=np.float32)
    lg = torch.from_numpy(np.log(gam)).view(1, 3, 1, 1).expand(2, 3, 500, 64).contiguous().cuda()
    og, sg = rc.gla_fwd(q, k, v, lg)
    orr, sr = rc.retention_fwd(q, k, v, gam, chunk=64)
    torch.cuda.synchronize()
    e_o = oracle.rel_frobenius(og.cpu().numpy(), orr.cpu().numpy())
    e_s = oracle.rel_frobenius(sg.cpu().numpy(), sr.cpu().numpy())
    print(f"[parity] gla constant gate vs retention_fwd: out {e_o:.3e} state {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("G", [1, 3, 7])
def test_gla_forced_segments(G, plan):
    plan(segments=G)
    w, inp = _inputs(78, 2, 2, 1000, 128, 64, 1.0)
    inp["lg"][:, :, 300:364] = -3.0  # one chunk's worth of strong gates inside a segment
    out, fs = _run(inp)
    _check(f"gla G={G}", out, fs, inp)


def test_gla_empty_and_zero_length():
    q = torch.zeros((1, 2, 0, 64), device="cuda")
    out, fs = rc.gla_fwd(q, q, q, q)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and torch.all(fs == 0)


def test_gla_mixed_gate_strength():
    """Strong gates (chunk sums below -80, the exact path) and weak ones (the
    fast path) alternating in one sequence."""
    w, inp = _inputs(76, 2, 2, 640, 64, 128, 2.0)
    g = torch.Generator().manual_seed(77)
    strong = torch.nn.functional.logsigmoid(torch.randn((2, 2, 640, 64), generator=g) - 2.5)
    for c0 in range(0, 640, 128):
        inp["lg"][:, :, c0:c0 + 64] = strong[:, :, c0:c0 + 64]
    out, fs = _run(inp)
    _check("gla mixed gate strength", out, fs, inp)


@pytest.mark.parametrize("mu", [3.0, -2.0])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 333), (128, 128, 300), (64, 128, 129), (128, 64, 200)])
def test_gla_bf16_small_full(mu, dk, dv, T):
    """bf16 q, k, v and out with fp32 gates; the oracle reads the rounded inputs."""
    w, inp = _inputs(81, 2, 3, T, dk, dv, mu, dtype="bf16")
    out, fs = _run(inp)
    _check(f"gla bf16 mu={mu} dk={dk} dv={dv} T={T}", out, fs, inp, tol=TOLS["bf16"])


@pytest.mark.parametrize("G", [1, 3])
def test_gla_bf16_segments_and_mixed_gates(G, plan):
    plan(segments=G)
    w, inp = _inputs(82, 2, 2, 700, 64, 64, 2.0, dtype="bf16")
    g = torch.Generator().manual_seed(83)
    strong = torch.nn.functional.logsigmoid(torch.randn((2, 2, 700, 64), generator=g) - 2.5)
    inp["lg"][:, :, 128:192] = strong[:, :, 128:192]  # one chunk on the exact path
    out, fs = _run(inp)
    _check(f"gla bf16 G={G} mixed", out, fs, inp, tol=TOLS["bf16"])


def test_gla_gates_above_one_are_taken_as_one():
    """A log-gate above 0 (a gate above 1) is outside the model; the kernel
    takes it as 0, so the result equals the oracle on the clamped gates."""
    w, inp = _inputs(84, 1, 2, 300, 64, 64, 1.0)
    lg = inp["lg"].clone()
    lg[:, :, 50:60] = 0.7
    lg[:, 1, 200, :7] = 3.0
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out, fs = rc.gla_fwd(q, k, v, lg.cuda())
    torch.cuda.synchronize()
    clamped = dict(inp, lg=torch.clamp(lg, max=0.0))
    _check("gla gates above one", out.cpu().numpy(), fs.cpu().numpy(), clamped)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gla_bench_shape(dtype):
    """[4, 8, 2048, 64] with log-sigmoid(N(2, 1)) gates, the benchmark's GLA workload, in full."""
    w, inp = _inputs(85, 4, 8, 2048, 64, 64, 2.0, dtype=dtype)
    out, fs = _run(inp)
    _check(f"gla [4,8,2048,64] {dtype}", out, fs, inp, tol=TOLS[dtype])
