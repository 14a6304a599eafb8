"""Segment-split forward (bf16) against the fp64 oracle (needs a gfx950 GPU).

The segment path cuts every (b, h) sequence into G segments: one kernel sums
each full segment's decayed k v^T contributions, the walk kernel starts each
segment from the decayed sum of the earlier ones.  These cases force the path
and the segment count through the library's plan override
(retention_set_plan_override) and compare out and the final state with the oracle in full: one and
several segments, segment counts that do not divide the chunk count, ragged
last chunks, chunk 64 and 128, every (dk, dv) pair, small and unit decays.
Tolerance: relative Frobenius error 2e-2 (bf16 inputs, fp32 accumulation).
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


def _inputs(seed, **over):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(**{"dtype": "bf16", **over})
    return w, wl.make_inputs(w, seed)


def _run(inp, chunk, plan, path="segment", segments=None):
    plan(path=path, segments=segments)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    print(f"[segment] chunk={chunk} path={path} G={segments} shape={tuple(q.shape)} dv={v.shape[-1]}",
          flush=True)
    out, fs = rc.retention_fwd(q, k, v, inp["gamma"], chunk=chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fs.cpu().numpy()


def _check(tag, out, fs, inp):
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    parity.check(f"{tag} out", out, ref, TOL)
    parity.check(f"{tag} state", fs, ref_s, TOL)


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, 1), (1000, 3), (1333, 4), (700, 16)])
def test_segment_small_full(chunk, dk, dv, T, G, plan):
    w, inp = _inputs(seed=11, B=2, H=2, T=T, dk=dk, dv=dv, chunk=chunk, scale=1.0 / np.sqrt(dk))
    out, fs = _run(inp, chunk, plan, segments=G)
    _check(f"segment C={chunk} dk={dk} dv={dv} T={T} G={G}", out, fs, inp)


@pytest.mark.parametrize("T", [1, 37, 128, 129, 255, 256, 257])
def test_segment_short_and_ragged(T, plan):
    w, inp = _inputs(seed=12, B=1, H=3, T=T, dk=128, dv=128, chunk=128, scale=1.0 / np.sqrt(128))
    out, fs = _run(inp, 128, plan, segments=2)
    _check(f"segment short T={T}", out, fs, inp)


def test_segment_zero_length(plan):
    w, inp = _inputs(seed=13, B=1, H=2, T=0, dk=128, dv=128, chunk=128)
    out, fs = _run(inp, 128, plan, segments=4)
    assert out.size == 0 and np.all(fs == 0.0)


@pytest.mark.parametrize("gval", [1.0, 0.5, 0.02])
def test_segment_gamma_extremes(gval, plan):
    w, inp = _inputs(seed=14, B=1, H=2, T=900, dk=64, dv=64, chunk=64, scale=1.0 / 8)
    inp["gamma"] = np.full(w.H, gval, dtype=np.float32)
    out, fs = _run(inp, 64, plan, segments=5)
    _check(f"segment gamma={gval}", out, fs, inp)


def test_segment_matches_slice_path_and_is_deterministic(plan):
    w, inp = _inputs(seed=15, B=1, H=4, T=2000, dk=128, dv=128, chunk=128, scale=1.0 / np.sqrt(128))
    o_seg, s_seg = _run(inp, 128, plan, segments=6)
    o_seg2, s_seg2 = _run(inp, 128, plan, segments=6)
    assert np.array_equal(o_seg, o_seg2) and np.array_equal(s_seg, s_seg2), "run-to-run results differ"
    o_sl, s_sl = _run(inp, 128, plan, path="slice")
    _check("segment G=6", o_seg, s_seg, inp)
    _check("slice", o_sl, s_sl, inp)
    e = oracle.rel_frobenius(o_seg, o_sl)
    print(f"[parity] segment vs slice out {e:.3e}", flush=True)
    assert e <= TOL


def test_segment_auto_choice(plan):
    # automatic segment count (several segments for 2 heads x 24 chunks)
    w, inp = _inputs(seed=16, B=1, H=2, T=3000, dk=128, dv=128, chunk=128, scale=1.0 / np.sqrt(128))
    out, fs = _run(inp, 128, plan, segments=None)
    _check("segment auto", out, fs, inp)


# ------------------------------------------------------------- elu+1 linear attention
def _run_lin(inp, plan, path="segment", segments=None):
    plan(path=path, segments=segments)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    print(f"[segment] linattn path={path} G={segments} shape={tuple(q.shape)} dv={v.shape[-1]}", flush=True)
    out = rc.linear_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check_lin(tag, out, inp):
    ref, _, _ = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    parity.check(f"{tag} out", out, ref, TOL)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, 1), (1333, 3), (2000, 8)])
def test_segment_linattn_full(dk, dv, T, G, plan):
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=2, H=2, T=T, dk=dk, dv=dv)
    inp = wl.make_inputs(w, 21)
    out = _run_lin(inp, plan, segments=G)
    _check_lin(f"linattn segment dk={dk} dv={dv} T={T} G={G}", out, inp)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129, 300])
def test_segment_linattn_short_and_ragged(T, plan):
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=1, H=3, T=T)
    inp = wl.make_inputs(w, 22)
    out = _run_lin(inp, plan, segments=2)
    _check_lin(f"linattn segment short T={T}", out, inp)


def test_segment_linattn_matches_slice_path(plan):
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=2, H=4, T=1500)
    inp = wl.make_inputs(w, 23)
    o_seg = _run_lin(inp, plan, segments=5)
    o_seg2 = _run_lin(inp, plan, segments=5)
    assert np.array_equal(o_seg, o_seg2), "run-to-run results differ"
    o_sl = _run_lin(inp, plan, path="slice")
    _check_lin("linattn segment G=5", o_seg, inp)
    _check_lin("linattn slice", o_sl, inp)
    e = oracle.rel_frobenius(o_seg, o_sl)
    print(f"[parity] linattn segment vs slice {e:.3e}", flush=True)
    assert e <= TOL


# ------------------------------------------------------------- caller workspace
def test_caller_workspace_contents_do_not_matter(plan):
    """A caller-owned workspace filled with garbage gives the same bits as a
    fresh one; a workspace one byte short is refused."""
    w, inp = _inputs(seed=17, B=1, H=4, T=4000, dk=128, dv=128, chunk=128, scale=1.0 / np.sqrt(128))
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    need = rc.retention_fwd_workspace_bytes(1, 4, 4000, 128, 128, 128, torch.bfloat16)
    print(f"[segment] caller workspace {need} bytes", flush=True)
    assert need > 0
    o1, s1 = rc.retention_fwd(q, k, v, inp["gamma"], chunk=128)
    ws = torch.full((need + 4096,), 0x7F, dtype=torch.uint8, device="cuda")
    o2, s2 = rc.retention_fwd(q, k, v, inp["gamma"], chunk=128, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    with pytest.raises(RuntimeError, match="RET_ERR_WORKSPACE"):
        rc.retention_fwd(q, k, v, inp["gamma"], chunk=128, workspace=ws[: need - 1])

    wa = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=1, H=4, T=4000)
    li = wl.make_inputs(wa, 24)
    lq, lk, lv = (li[n].cuda() for n in ("q", "k", "v"))
    lneed = rc.linear_attn_workspace_bytes(1, 4, 4000, wa.dk, wa.dv, torch.bfloat16)
    assert lneed > 0
    l1 = rc.linear_attn_fwd(lq, lk, lv)
    lws = torch.full((lneed,), 0xFF, dtype=torch.uint8, device="cuda")
    l2 = rc.linear_attn_fwd(lq, lk, lv, workspace=lws)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)


# ------------------------------------------------------------- segmented value-slice walk
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, 2), (1333, 5), (700, 16)])
def test_slice_segments_full(dtype, chunk, dk, dv, T, G, plan):
    """The value-slice walk split into G segments (fp32 picks G by itself;
    bf16 only when forced), against the oracle in full."""
    w, inp = _inputs(seed=18, B=2, H=2, T=T, dk=dk, dv=dv, chunk=chunk, scale=1.0 / np.sqrt(dk), dtype=dtype)
    out, fs = _run(inp, chunk, plan, path="slice", segments=G)
    tol = 1e-4 if dtype == "f32" else TOL
    ref, ref_s = oracle.retention_recurrent(inp["q"], inp["k"], inp["v"], inp["gamma"], nthreads=8)
    e_o, e_s = oracle.rel_frobenius(out, ref), oracle.rel_frobenius(fs, ref_s)
    print(f"[parity] slice {dtype} C={chunk} dk={dk} dv={dv} T={T} G={G}: out {e_o:.3e} state {e_s:.3e}", flush=True)
    assert e_o <= tol and e_s <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("T,G", [(1000, 3), (300, 16)])
def test_slice_segments_linattn(dtype, dk, dv, T, G, plan):
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype)
    inp = wl.make_inputs(w, 25)
    out = _run_lin(inp, plan, path="slice", segments=G)
    ref, _, _ = oracle.linattn_recurrent(inp["q"], inp["k"], inp["v"], nthreads=8)
    e = oracle.rel_frobenius(out, ref)
    tol = 1e-4 if dtype == "f32" else TOL
    print(f"[parity] slice linattn {dtype} dk={dk} dv={dv} T={T} G={G}: {e:.3e}", flush=True)
    assert e <= tol and np.isfinite(out).all()


def test_f32_auto_segments_match_one_segment(plan):
    """fp32 automatic segments against the forced single-segment walk."""
    w, inp = _inputs(seed=19, B=4, H=8, T=2048, dk=64, dv=64, chunk=64, scale=1.0 / 8, dtype="f32")
    o_auto, s_auto = _run(inp, 64, plan, path="slice", segments=None)
    o_one, s_one = _run(inp, 64, plan, path="slice", segments=1)
    e_o, e_s = oracle.rel_frobenius(o_auto, o_one), oracle.rel_frobenius(s_auto, s_one)
    print(f"[parity] f32 auto vs one segment: out {e_o:.3e} state {e_s:.3e}", flush=True)
    assert e_o <= 1e-5 and e_s <= 1e-5
