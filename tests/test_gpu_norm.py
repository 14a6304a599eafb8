"""Retention with the row-sum floor and GroupNorm fused into the walk
(retention_fwd_normalized) against the fp64 oracle (needs a gfx950 GPU).

The oracle follows the normaliser recurrence n_t = gamma n_{t-1} + k_t and
divides each read-out by max(|n_t . q_t|, 1), then standardises each row for
GroupNorm.  Cases: both normalisations, chunks 64 and 128, every (dk, dv)
pair, several segment counts, ragged and short lengths, decays from 0.02 to 1,
inputs scaled so that the floor is active for some rows and not for others,
and the long bf16 shape on sampled heads.  The fp32 value-slice walk is held
to the same oracle on every shape it takes.  Tolerance: relative Frobenius
error 2e-2 (bf16 inputs, fp32 accumulation, one bf16 rounding), 1e-4 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL32 = 1e-4


def _inputs(seed, B, H, T, dk, dv, qscale=1.0, dtype="bf16"):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, scale=1.0)
    inp = wl.make_inputs(w, seed)
    tdt = wl.torch_dtype(dtype)
    # q scaled so the score row sums straddle the floor of 1
    inp["q"] = (inp["q"].float() * (qscale / np.sqrt(dk))).to(tdt)
    inp["k"] = (inp["k"].float() / np.sqrt(dk)).to(tdt)
    return w, inp


def _run(inp, norm, chunk, plan, G=None, eps=1e-5):
    plan(segments=G)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out = rc.retention_fwd_normalized(q, k, v, inp["gamma"], norm=norm, eps=eps, chunk=chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check(tag, out, inp, norm, eps=1e-5, tol=TOL):
    ref = oracle.retention_normalized(inp["q"], inp["k"], inp["v"], inp["gamma"], group=(norm == "group"), eps=eps,
                                      nthreads=8)
    parity.check(tag, out, ref, tol)


@pytest.mark.parametrize("norm", ["rowsum", "group"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, None), (1333, 4), (300, 1)])
def test_norm_small_full(norm, chunk, dk, dv, T, G, plan):
    w, inp = _inputs(61, 2, 3, T, dk, dv, qscale=2.0)
    out = _run(inp, norm, chunk, plan, G)
    _check(f"norm {norm} C={chunk} dk={dk} dv={dv} T={T} G={G}", out, inp, norm)


@pytest.mark.parametrize("norm", ["rowsum", "group"])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 129])
def test_norm_short_and_ragged(norm, T, plan):
    w, inp = _inputs(62, 1, 2, T, 64, 64, qscale=3.0)
    out = _run(inp, norm, 64, plan, 2)
    _check(f"norm {norm} short T={T}", out, inp, norm)


@pytest.mark.parametrize("gval", [1.0, 0.5, 0.02])
@pytest.mark.parametrize("qscale", [0.05, 20.0])
def test_norm_gamma_and_floor(gval, qscale, plan):
    """Small q keeps every row sum under the floor (output = plain retention,
    then GroupNorm); large q puts every row past it."""
    w, inp = _inputs(63, 1, 2, 900, 64, 64, qscale=qscale)
    inp["gamma"] = np.full(2, gval, dtype=np.float32)
    for norm in ("rowsum", "group"):
        out = _run(inp, norm, 64, plan, 3)
        # gamma = 1 with large q: signed scores cancel in the row sum, so the
        # divisor must come from the fp32 scores, not the bf16 P operand
        # (summed from bf16 weights this case reached 1.24e-2)
        tol = 6e-3 if (norm == "rowsum" and gval == 1.0 and qscale == 20.0) else TOL
        _check(f"norm {norm} gamma={gval} qscale={qscale}", out, inp, norm, tol=tol)


def test_norm_group_eps(plan):
    w, inp = _inputs(64, 1, 2, 500, 64, 64, qscale=2.0)
    out = _run(inp, "group", 64, plan, None, eps=0.5)
    _check("norm group eps=0.5", out, inp, "group", eps=0.5)


def test_norm_long_sequence_whole_tensor(plan):
    """[1, 32, 65536, 128] bf16 with the floor and GroupNorm: every row of
    every head against the oracle, 8 heads at a time."""
    w = wl.WORKLOADS["ret_fwd_long_bf16"]
    inp = wl.make_inputs(w, 0)
    out = _run(inp, "group", 128, plan, None)
    acc = parity.HeadGroups("norm group long [1,32,65536,128]", TOL)
    for h0 in range(0, w.H, 8):
        sl = (slice(None), slice(h0, h0 + 8))
        ref = oracle.retention_normalized(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["gamma"][h0:h0 + 8],
                                          group=True, eps=1e-5, nthreads=16)
        acc.add(out[sl], ref, h0)
    acc.finish()


def _offset_inputs(seed, B, H, T, dk, dv, offset, dtype):
    """Queries and keys near 0.5 (every score positive, every row sum far past
    the floor), gamma = 0.5: each read-out is a decayed weighted mean of the
    values offset + N(0, 1), so the rows GroupNorm standardises have a mean
    near `offset` and a spread under 1, where E[x^2] - mean^2 cancels."""
    g = torch.Generator().manual_seed(seed)
    tdt = wl.torch_dtype(dtype)
    q = (0.5 + 0.1 * torch.randn((B, H, T, dk), generator=g)).to(tdt)
    k = (0.5 + 0.1 * torch.randn((B, H, T, dk), generator=g)).to(tdt)
    v = (offset + torch.randn((B, H, T, dv), generator=g)).to(tdt)
    return {"q": q, "k": k, "v": v, "gamma": np.full(H, 0.5, dtype=np.float32)}


@pytest.mark.parametrize("chunk,dk,dv", [(64, 64, 64), (128, 128, 128), (64, 128, 64)])
def test_norm_group_rows_with_large_mean(chunk, dk, dv, plan):
    """bf16 segment walk, values offset by 100 (bf16 keeps 0.5 steps there):
    rows with a mean near 100 standardise within the bf16 tolerance.  (A
    larger offset would measure the bf16 rounding of the state copy that the
    inter-chunk product reads, not the row statistics.)"""
    inp = _offset_inputs(65, 2, 3, 700, dk, dv, 100.0, "bf16")
    out = _run(inp, "group", chunk, plan, 3)
    _check(f"norm group offset 100 C={chunk} dk={dk} dv={dv}", out, inp, "group")


def test_norm_group_zero_query_rows_are_zero(plan):
    """Tokens with q = 0 have an all-zero read-out; GroupNorm with eps > 0
    maps that row to zeros, in both dtypes."""
    for dtype, tol in (("bf16", TOL), ("f32", TOL32)):
        w, inp = _inputs(66, 1, 2, 400, 64, 64, qscale=2.0, dtype=dtype)
        q = inp["q"].clone()
        q[:, :, 100:164] = 0
        q[:, :, 399] = 0
        inp["q"] = q
        out = _run(inp, "group", 64, plan, 2)
        assert np.all(out[:, :, 100:164] == 0) and np.all(out[:, :, 399] == 0)
        _check(f"norm group zero query rows {dtype}", out, inp, "group", tol=tol)


# ---------------------------------------------------------------- fp32 (value-slice walk)
F32_GROUP_SHAPES = [(64, 64, 64), (64, 64, 128), (64, 128, 64), (128, 64, 64)]  # (chunk, dk, dv)


@pytest.mark.parametrize("chunk,dk,dv", F32_GROUP_SHAPES)
@pytest.mark.parametrize("T,G", [(1000, None), (1333, 4), (300, 1)])
def test_norm_f32_group(chunk, dk, dv, T, G, plan):
    w, inp = _inputs(71, 2, 3, T, dk, dv, qscale=2.0, dtype="f32")
    out = _run(inp, "group", chunk, plan, G)
    _check(f"norm f32 group C={chunk} dk={dk} dv={dv} T={T} G={G}", out, inp, "group", tol=TOL32)


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, None), (1333, 4)])
def test_norm_f32_rowsum(chunk, dk, dv, T, G, plan):
    w, inp = _inputs(72, 2, 3, T, dk, dv, qscale=2.0, dtype="f32")
    out = _run(inp, "rowsum", chunk, plan, G)
    _check(f"norm f32 rowsum C={chunk} dk={dk} dv={dv} T={T} G={G}", out, inp, "rowsum", tol=TOL32)


@pytest.mark.parametrize("norm", ["rowsum", "group"])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 129])
def test_norm_f32_short_and_ragged(norm, T, plan):
    w, inp = _inputs(73, 1, 2, T, 64, 64, qscale=3.0, dtype="f32")
    out = _run(inp, norm, 64, plan, 2)
    _check(f"norm f32 {norm} short T={T}", out, inp, norm, tol=TOL32)


@pytest.mark.parametrize("gval", [1.0, 0.5, 0.02])
@pytest.mark.parametrize("qscale", [0.05, 20.0])
def test_norm_f32_gamma_and_floor(gval, qscale, plan):
    w, inp = _inputs(74, 1, 2, 900, 64, 64, qscale=qscale, dtype="f32")
    inp["gamma"] = np.full(2, gval, dtype=np.float32)
    for norm in ("rowsum", "group"):
        out = _run(inp, norm, 64, plan, 3)
        _check(f"norm f32 {norm} gamma={gval} qscale={qscale}", out, inp, norm, tol=TOL32)


@pytest.mark.parametrize("chunk,dk,dv", [(64, 128, 128), (128, 64, 128), (128, 128, 64), (128, 128, 128)])
@pytest.mark.parametrize("T,G", [(1000, None), (700, 3)])
def test_norm_f32_group_rows_over_slices(chunk, dk, dv, T, G, plan):
    """Shapes whose rows span several value slices: the walk applies the floor
    and a row pass standardises in place."""
    w, inp = _inputs(75, 2, 3, T, dk, dv, qscale=2.0, dtype="f32")
    out = _run(inp, "group", chunk, plan, G)
    _check(f"norm f32 group (row pass) C={chunk} dk={dk} dv={dv} T={T} G={G}", out, inp, "group", tol=TOL32)


@pytest.mark.parametrize("chunk,dk,dv", F32_GROUP_SHAPES + [(64, 128, 128), (128, 128, 128)])
def test_norm_f32_group_rows_with_large_mean(chunk, dk, dv, plan):
    """fp32, values offset by 100, on the fused shapes and on shapes that take
    the row pass: rows with a mean near 100 and a spread under 1 keep the
    fp32 tolerance (two-pass statistics)."""
    inp = _offset_inputs(76, 2, 3, 700, dk, dv, 100.0, "f32")
    out = _run(inp, "group", chunk, plan, 3)
    _check(f"norm f32 group offset 100 C={chunk} dk={dk} dv={dv}", out, inp, "group", tol=TOL32)
